"""Seeded synthetic inputs for the routed-expert MoE layer.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It draws random numbers and lays them out in the packed byte
formats; it performs none of the layer's arithmetic (no decoding, no routing,
no matrix products).

Shapes follow the MiMo-V2.6-Flash-RL model cards: each token is routed to 8 of
256 experts, with no shared expert (TrevorJS GGUF card, "Architecture notes"); expert
intermediate width 2048 (Baekpica VQ card, "Why 13 bits plus an 8-bit
residual"); hidden width 4096 (implied by the routed-parameter and payload
totals on the savrn mixed-quant card, "Memory metrics").  Experts are stored as
MXFP4 (TrevorJS card, "Architecture notes": one E8M0 exponent per 32 values) or
as 8-dimensional VQ codes (Baekpica VQ card, "Recipe").

Randomness: numpy PCG64 seeded through ``SeedSequence(seed).spawn``, one child
stream per tensor, so every tensor is reproducible on its own.

Packed formats (the byte layout is this project's own; the pages fix only the
element encodings):

MXFP4 layer = E experts back to back, each ``mxfp4_expert_bytes(H, I)`` bytes:
  [gate/up codes][gate/up scales][down codes][down scales]
  gate/up is one matrix of 2I rows (rows 0..I-1 gate, I..2I-1 up) by H columns;
  down is H rows by I columns.  A matrix of N rows and K columns is cut into
  tiles of 16 rows x 32 columns, stored tile after tile, tile (a, b) at index
  a*(K/32) + b.  A tile holds 256 code bytes (row r of the tile at bytes
  16r..16r+15, column c in byte c/2, even c in the low nibble) and, in the
  scale region, 16 E8M0 bytes (one per row of the tile).

VQ13R8 layer = [Cb 8192x8 fp16][Rb 256x8 fp16] then E experts, each
``vq_expert_bytes(H, I)`` bytes:
  [gu code12][gu plane][gu res][gu gain][dn code12][dn plane][dn res][dn gain]
  A matrix of N rows by K columns has N*K/8 vectors of 8 consecutive columns.
  Tiles are 16 rows x 256 columns (512 vectors), tile (a, b) at a*(K/256)+b.
  Inside a tile vector (row r, column 8*j) has stream position
  ((j // 8) * 16 + r) * 8 + (j % 8).  code12 is a little-endian 12-bit stream
  over stream positions, plane a little-endian bit stream, res a byte stream.
  gains are one fp16 per matrix row, in row order.
"""

from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

FMT_MXFP4 = 1
FMT_VQ13R8 = 2
FMT_VQ13 = 3
VQ_FORMATS = (FMT_VQ13R8, FMT_VQ13)

VQ_BOOK_ENTRIES = 8192
VQ_RES_ENTRIES = 256
VQ_DIM = 8
VQ_BOOKS_BYTES = (VQ_BOOK_ENTRIES + VQ_RES_ENTRIES) * VQ_DIM * 2
VQ13_BOOKS_BYTES = VQ_BOOK_ENTRIES * VQ_DIM * 2


# ---------------------------------------------------------------------------
# byte sizes of the packed formats
# ---------------------------------------------------------------------------

def mxfp4_matrix_regions(n: int, k: int) -> tuple[int, int]:
    """(code bytes, scale bytes) of one MXFP4 matrix of n rows by k columns."""
    return n * k // 2, n * k // 32


def mxfp4_expert_regions(h: int, i: int) -> dict[str, tuple[int, int]]:
    """Byte ranges [start, stop) of the four regions inside one MXFP4 expert."""
    gc, gs = mxfp4_matrix_regions(2 * i, h)
    dc, ds = mxfp4_matrix_regions(h, i)
    out, off = {}, 0
    for name, size in (("gu_codes", gc), ("gu_scales", gs), ("dn_codes", dc), ("dn_scales", ds)):
        out[name] = (off, off + size)
        off += size
    return out


def mxfp4_expert_bytes(h: int, i: int) -> int:
    return mxfp4_expert_regions(h, i)["dn_scales"][1]


def vq_matrix_regions(n: int, k: int, res: bool = True) -> tuple[int, int, int, int]:
    """(code12, plane, res, gain) byte counts of one VQ matrix (res 0 for VQ13)."""
    nvec = n * k // VQ_DIM
    return nvec * 3 // 2, nvec // 8, nvec if res else 0, n * 2


def vq_expert_regions(h: int, i: int, res: bool = True) -> dict[str, tuple[int, int]]:
    out, off = {}, 0
    for prefix, (n, k) in (("gu", (2 * i, h)), ("dn", (h, i))):
        c, p, r, g = vq_matrix_regions(n, k, res)
        for name, size in (("code12", c), ("plane", p), ("res", r), ("gain", g)):
            if size:
                out[f"{prefix}_{name}"] = (off, off + size)
            off += size
    return out


def vq_expert_bytes(h: int, i: int, res: bool = True) -> int:
    return vq_expert_regions(h, i, res)["dn_gain"][1]


def packed_bytes(fmt: int, h: int, i: int, e: int) -> int:
    if fmt == FMT_MXFP4:
        return e * mxfp4_expert_bytes(h, i)
    if fmt == FMT_VQ13R8:
        return VQ_BOOKS_BYTES + e * vq_expert_bytes(h, i)
    if fmt == FMT_VQ13:
        return VQ13_BOOKS_BYTES + e * vq_expert_bytes(h, i, res=False)
    raise ValueError(f"unknown format {fmt}")


def vq13_from_vq13r8(packed: np.ndarray, h: int, i: int, e: int) -> np.ndarray:
    """The VQ13 buffer holding the same 13-bit stage as a VQ13R8 buffer: the
    residual book and the residual index regions dropped, every other byte
    kept in order (byte slicing only)."""
    full = vq_expert_regions(h, i, True)
    ex = packed[VQ_BOOKS_BYTES:].reshape(e, vq_expert_bytes(h, i, True))
    keep = [ex[:, a:b] for name, (a, b) in full.items() if not name.endswith("_res")]
    return np.concatenate([packed[:VQ13_BOOKS_BYTES], np.concatenate(keep, axis=1).reshape(-1)])


# ---------------------------------------------------------------------------
# workload descriptions
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    hidden: int
    inter: int
    experts: int
    top_k: int
    fmt: int = FMT_MXFP4
    seed: int = 0
    # MXFP4 exponent range, inclusive
    exp_lo: int = 120
    exp_hi: int = 126
    # router skew: this many seeded "hot" experts get their router rows scaled
    hot_experts: int = 0
    hot_scale: float = 1.0
    # this many seeded tokens are multiplied by token_scale (exact in bf16)
    scaled_tokens: int = 0
    token_scale: float = 1.0
    router_std: float = 0.02
    # routing weights: 0 softmax over the selected logits, 1 normalised sigmoids
    routing: int = 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def routes(self) -> int:
        return self.tokens * self.top_k

    @property
    def packed_bytes(self) -> int:
        return packed_bytes(self.fmt, self.hidden, self.inter, self.experts)


# Tiny layer: correctness only.
TINY = Workload("tiny", tokens=16, hidden=256, inter=128, experts=8, top_k=2, seed=1)
# MiMo-shaped layer, decode batch 1.
DECODE = Workload("mimo_decode_t1", tokens=1, hidden=4096, inter=2048, experts=256, top_k=8, seed=2)
# 16-token verify batch with skewed routing: 32 hot experts take half the routes.
VERIFY = Workload("mimo_verify_t16_skewed", tokens=16, hidden=4096, inter=2048, experts=256,
                  top_k=8, seed=3, hot_experts=32, hot_scale=1.845)
# 2048-token prefill micro-batch; 20 tokens (1%) scaled by 64 so that SwiGLU
# intermediates exceed the fp16 range.
PREFILL = Workload("mimo_prefill_t2048", tokens=2048, hidden=4096, inter=2048, experts=256,
                   top_k=8, seed=4, scaled_tokens=20, token_scale=64.0)
# VQ R13+8 experts, 2048 tokens.
VQ_PREFILL = Workload("mimo_vq_prefill_t2048", tokens=2048, hidden=4096, inter=2048,
                      experts=256, top_k=8, fmt=FMT_VQ13R8, seed=5)
# Test-only tiny VQ layer (VQ tiles need multiples of 256 in both widths).
TINY_VQ = Workload("tiny_vq", tokens=16, hidden=256, inter=256, experts=8, top_k=2,
                   fmt=FMT_VQ13R8, seed=6)
# the 13-bit stage alone (every VQ layer has it; 32 of 48 add the residual)
TINY_VQ13 = TINY_VQ.replace(name="tiny_vq13", fmt=FMT_VQ13, seed=7)
VQ13_DECODE = Workload("mimo_vq13_decode_t1", tokens=1, hidden=4096, inter=2048, experts=256,
                       top_k=8, fmt=FMT_VQ13, seed=8)

PRESETS = {w.name: w for w in (TINY, DECODE, VERIFY, PREFILL, VQ_PREFILL, TINY_VQ, TINY_VQ13,
                               VQ13_DECODE)}

# stream numbers inside SeedSequence(seed).spawn(N_STREAMS)
_S_X, _S_ROUTER, _S_CODES, _S_SCALES, _S_HOT, _S_SCALED, _S_BOOKS, _S_GAINS = range(8)
_N_STREAMS = 8


def _streams(seed: int) -> list[np.random.Generator]:
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(_N_STREAMS)]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the
    16-bit patterns.  Input preparation only (the layer receives bf16)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_x(w: Workload, tokens: Optional[int] = None, stream_offset: int = 0) -> np.ndarray:
    """Activations x [T, H] as bf16 bit patterns (uint16): bf16(N(0,1)); the
    workload's scaled tokens are multiplied by token_scale (a power of two, so
    the scaling is exact).  ``stream_offset`` selects an independent batch of
    the same distribution (used for fresh tokens per benchmark step)."""
    t = w.tokens if tokens is None else tokens
    rs = _streams(w.seed + 1_000_003 * stream_offset)
    x = rs[_S_X].standard_normal((t, w.hidden), dtype=np.float32)
    if w.scaled_tokens:
        sel = rs[_S_SCALED].choice(t, size=min(w.scaled_tokens, t), replace=False)
        x[sel] *= np.float32(w.token_scale)
    return f32_to_bf16_bits(x)


def scaled_token_ids(w: Workload, tokens: Optional[int] = None, stream_offset: int = 0) -> np.ndarray:
    t = w.tokens if tokens is None else tokens
    if not w.scaled_tokens:
        return np.zeros(0, dtype=np.int64)
    rs = _streams(w.seed + 1_000_003 * stream_offset)
    rs[_S_X].standard_normal((t, w.hidden), dtype=np.float32)  # keep stream positions aligned
    return np.sort(rs[_S_SCALED].choice(t, size=min(w.scaled_tokens, t), replace=False))


def make_router(w: Workload) -> np.ndarray:
    """Router weights W_r [E, H] float32 ~ N(0, router_std); hot experts'
    rows are multiplied by hot_scale."""
    rs = _streams(w.seed)
    r = (rs[_S_ROUTER].standard_normal((w.experts, w.hidden), dtype=np.float32)
         * np.float32(w.router_std))
    if w.hot_experts:
        hot = rs[_S_HOT].choice(w.experts, size=w.hot_experts, replace=False)
        r[hot] *= np.float32(w.hot_scale)
    return np.ascontiguousarray(r)


def hot_expert_ids(w: Workload) -> np.ndarray:
    if not w.hot_experts:
        return np.zeros(0, dtype=np.int64)
    rs = _streams(w.seed)
    return np.sort(rs[_S_HOT].choice(w.experts, size=w.hot_experts, replace=False))


def make_experts(w: Workload) -> np.ndarray:
    """The packed expert buffer (uint8) of the workload's format."""
    if w.fmt == FMT_MXFP4:
        return _make_mxfp4(w)
    if w.fmt in VQ_FORMATS:
        return _make_vq(w)
    raise ValueError(w.fmt)


def _make_mxfp4(w: Workload) -> np.ndarray:
    rs = _streams(w.seed)
    s = mxfp4_expert_bytes(w.hidden, w.inter)
    # Uniform bytes give two independent uniform 4-bit codes per byte.
    buf = rs[_S_CODES].integers(0, 256, size=(w.experts, s), dtype=np.uint8)
    reg = mxfp4_expert_regions(w.hidden, w.inter)
    for name in ("gu_scales", "dn_scales"):
        a, b = reg[name]
        buf[:, a:b] = rs[_S_SCALES].integers(w.exp_lo, w.exp_hi + 1, size=(w.experts, b - a),
                                             dtype=np.uint8)
    return buf.reshape(-1)


def _make_vq(w: Workload) -> np.ndarray:
    res = w.fmt == FMT_VQ13R8
    rs = _streams(w.seed)
    entries = VQ_BOOK_ENTRIES + (VQ_RES_ENTRIES if res else 0)
    books = rs[_S_BOOKS].standard_normal((entries * VQ_DIM,), dtype=np.float32).astype(np.float16)
    s = vq_expert_bytes(w.hidden, w.inter, res)
    # Uniform bytes give uniform 12-bit codes, plane bits and residual indices.
    ex = rs[_S_CODES].integers(0, 256, size=(w.experts, s), dtype=np.uint8)
    reg = vq_expert_regions(w.hidden, w.inter, res)
    for name, k in (("gu_gain", w.hidden), ("dn_gain", w.inter)):
        a, b = reg[name]
        rows = (b - a) // 2
        g = rs[_S_GAINS].uniform(0.5, 1.5, size=(w.experts, rows)) / np.sqrt(2.0 * k)
        ex[:, a:b] = g.astype(np.float16).view(np.uint8).reshape(w.experts, b - a)
    return np.concatenate([books.view(np.uint8), ex.reshape(-1)])


def make_zero_experts(w: Workload) -> np.ndarray:
    return np.zeros(w.packed_bytes, dtype=np.uint8)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()
