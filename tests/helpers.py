"""Test helpers: an independent numpy packer/unpacker for the packed formats,
a dense numpy evaluator of the layer, and the output tolerance check.

These are written separately from the C oracle (vectorised numpy instead of
per-element C) so that the tests can pin the oracle against them.
"""

from __future__ import annotations

import math

import numpy as np

import workloads as W

# OCP MX v1.0 E2M1 table, read from tests/golden/e2m1_table.txt by the tests.
_E2M1 = None


def e2m1_table() -> np.ndarray:
    global _E2M1
    if _E2M1 is None:
        import os
        vals = np.zeros(16, dtype=np.float64)
        path = os.path.join(os.path.dirname(__file__), "golden", "e2m1_table.txt")
        with open(path) as f:
            for line in f:
                line = line.strip()
                if not line or line.startswith("#"):
                    continue
                c, v = line.split()
                vals[int(c)] = float(v)
        _E2M1 = vals
    return _E2M1


# ---------------------------------------------------------------------------
# MXFP4 tiles: 16 rows x 32 columns
# ---------------------------------------------------------------------------

def mx_pack(codes: np.ndarray, scales: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """codes [N, K] (0..15), scales [N, K/32] (0..255) -> tiled code bytes and
    scale bytes."""
    n, k = codes.shape
    c = codes.astype(np.uint8).reshape(n // 16, 16, k // 32, 16, 2)   # a, r, b, byte, nibble
    byte = c[..., 0] | (c[..., 1] << 4)                                  # a, r, b, byte
    code_bytes = byte.transpose(0, 2, 1, 3).reshape(-1)                  # a, b, r, byte
    s = scales.astype(np.uint8).reshape(n // 16, 16, k // 32)            # a, r, b
    scale_bytes = s.transpose(0, 2, 1).reshape(-1)                       # a, b, r
    return np.ascontiguousarray(code_bytes), np.ascontiguousarray(scale_bytes)


def mx_unpack(code_bytes: np.ndarray, scale_bytes: np.ndarray, n: int, k: int):
    """Inverse of mx_pack: (codes [N, K], scales [N, K/32])."""
    b = code_bytes.reshape(n // 16, k // 32, 16, 16).transpose(0, 2, 1, 3)  # a, r, b, byte
    lo = b & 15
    hi = b >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(n, k)
    s = scale_bytes.reshape(n // 16, k // 32, 16).transpose(0, 2, 1).reshape(n, k // 32)
    return codes, s


def mx_dense(code_bytes, scale_bytes, n, k) -> np.ndarray:
    codes, s = mx_unpack(code_bytes, scale_bytes, n, k)
    vals = e2m1_table()[codes]
    sc = np.ldexp(1.0, s.astype(np.int64) - 127).astype(np.float64)
    return vals * np.repeat(sc, 32, axis=1)


def mx_expert_dense(wl: W.Workload, packed: np.ndarray, e: int):
    """(gate [I,H], up [I,H], down [H,I]) in float64 for MXFP4 expert e."""
    h, i = wl.hidden, wl.inter
    s = W.mxfp4_expert_bytes(h, i)
    reg = W.mxfp4_expert_regions(h, i)
    ex = packed[e * s:(e + 1) * s]
    seg = {name: ex[a:b] for name, (a, b) in reg.items()}
    gu = mx_dense(seg["gu_codes"], seg["gu_scales"], 2 * i, h)
    dn = mx_dense(seg["dn_codes"], seg["dn_scales"], h, i)
    return gu[:i], gu[i:], dn


def mx_pack_expert(wl: W.Workload, gu_codes, gu_scales, dn_codes, dn_scales) -> np.ndarray:
    a, b = mx_pack(gu_codes, gu_scales)
    c, d = mx_pack(dn_codes, dn_scales)
    return np.concatenate([a, b, c, d])


# ---------------------------------------------------------------------------
# VQ tiles: 16 rows x 256 columns, 512 vectors
# ---------------------------------------------------------------------------

def vq_positions(n: int, k: int) -> np.ndarray:
    """Stream position of every vector [N, K/8] of an N x K VQ matrix."""
    rows = np.arange(n)[:, None]
    cols = np.arange(k // 8)[None, :]
    a, r = rows // 16, rows % 16
    b, jj = cols // 32, cols % 32
    tile = a * (k // 256) + b
    return tile * 512 + ((jj // 8) * 16 + r) * 8 + (jj % 8)


def vq_pack(i13: np.ndarray, i8: np.ndarray, gains_f16: np.ndarray):
    """i13 [N, K/8] (0..8191), i8 [N, K/8], gains [N] float16 -> (code12,
    plane, res, gain bytes)."""
    n, nv = i13.shape
    pos = vq_positions(n, nv * 8).reshape(-1)
    flat13 = np.empty(n * nv, dtype=np.int64)
    flat13[pos] = i13.reshape(-1)
    flat8 = np.empty(n * nv, dtype=np.uint8)
    flat8[pos] = i8.reshape(-1)
    c12 = flat13 & 0xFFF
    plane_bits = (flat13 >> 12) & 1
    # 12-bit little-endian stream: two codes per 3 bytes
    pair = c12.reshape(-1, 2)
    b0 = pair[:, 0] & 0xFF
    b1 = (pair[:, 0] >> 8) | ((pair[:, 1] & 0xF) << 4)
    b2 = pair[:, 1] >> 4
    code12 = np.stack([b0, b1, b2], axis=1).astype(np.uint8).reshape(-1)
    plane = np.packbits(plane_bits.astype(np.uint8), bitorder="little")
    return code12, plane, flat8, gains_f16.astype(np.float16).view(np.uint8)


def vq_unpack(code12, plane, res, n, k):
    """-> (i13 [N, K/8], i8 [N, K/8])."""
    pos = vq_positions(n, k)
    t = code12.reshape(-1, 3).astype(np.int64)
    c0 = t[:, 0] | ((t[:, 1] & 0xF) << 8)
    c1 = (t[:, 1] >> 4) | (t[:, 2] << 4)
    c12 = np.stack([c0, c1], axis=1).reshape(-1)
    bits = np.unpackbits(plane, bitorder="little").astype(np.int64)
    i13 = c12[pos] | (bits[pos] << 12)
    return i13, res[pos]


def vq_books(packed: np.ndarray):
    cb = packed[:8192 * 16].view(np.float16).reshape(8192, 8).astype(np.float64)
    rb = packed[8192 * 16:W.VQ_BOOKS_BYTES].view(np.float16).reshape(256, 8).astype(np.float64)
    return cb, rb


def vq_matrix_dense(packed: np.ndarray, base: int, n: int, k: int) -> tuple[np.ndarray, int]:
    c, p, r, g = W.vq_matrix_regions(n, k)
    off = base
    code12 = packed[off:off + c]; off += c
    plane = packed[off:off + p]; off += p
    res = packed[off:off + r]; off += r
    gain = packed[off:off + g].view(np.float16).astype(np.float64); off += g
    i13, i8 = vq_unpack(code12, plane, res, n, k)
    cb, rb = vq_books(packed)
    vec = cb[i13] + rb[i8]                       # [N, K/8, 8]
    return gain[:, None] * vec.reshape(n, k), off


def vq_expert_dense(wl: W.Workload, packed: np.ndarray, e: int):
    h, i = wl.hidden, wl.inter
    base = W.VQ_BOOKS_BYTES + e * W.vq_expert_bytes(h, i)
    gu, off = vq_matrix_dense(packed, base, 2 * i, h)
    dn, _ = vq_matrix_dense(packed, off, h, i)
    return gu[:i], gu[i:], dn


def expert_dense(wl: W.Workload, packed: np.ndarray, e: int):
    if wl.fmt == W.FMT_MXFP4:
        return mx_expert_dense(wl, packed, e)
    return vq_expert_dense(wl, packed, e)


# ---------------------------------------------------------------------------
# dense evaluator and tolerance
# ---------------------------------------------------------------------------

def silu_np(g: np.ndarray) -> np.ndarray:
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = g[pos] / (1.0 + np.exp(-g[pos]))
    z = np.exp(g[~pos])
    out[~pos] = g[~pos] * z / (1.0 + z)
    return out


def dense_ffn(gate, up, down, x: np.ndarray) -> np.ndarray:
    """SwiGLU MLP in float64 with numpy matmuls; x [T, H] float64."""
    g = x @ gate.T
    u = x @ up.T
    return (silu_np(g) * u) @ down.T


def check_output(got: np.ndarray, ref: np.ndarray, rel_l2: float = 2e-3, rel_max: float = 1e-2):
    """Per token row t: ||d_t||_2 <= rel_l2 * ||ref_t||_2 and
    max_j |d_tj| <= rel_max * rms(ref_t).  Returns (worst l2 ratio, worst
    max ratio); raises AssertionError on failure."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output"
    d = got - ref
    n_ref = np.linalg.norm(ref, axis=1)
    rms = n_ref / math.sqrt(ref.shape[1])
    n_d = np.linalg.norm(d, axis=1)
    m_d = np.abs(d).max(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        l2r = np.where(n_ref > 0, n_d / n_ref, np.where(n_d > 0, np.inf, 0.0))
        mxr = np.where(rms > 0, m_d / rms, np.where(m_d > 0, np.inf, 0.0))
    bad = np.nonzero((l2r > rel_l2) | (mxr > rel_max))[0]
    assert bad.size == 0, (f"{bad.size} rows out of tolerance, first rows {bad[:8].tolist()}: "
                           f"l2 {l2r[bad[:8]].tolist()} max {mxr[bad[:8]].tolist()}")
    return float(l2r.max(initial=0.0)), float(mxr.max(initial=0.0))
