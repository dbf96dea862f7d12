"""Pins of the oracle's element decoders and packed layouts (CPU only)."""

import math

import numpy as np
import pytest

import workloads as W
from helpers import e2m1_table, mx_pack, mx_unpack, vq_pack, vq_unpack, vq_positions


def test_e2m1_matches_ocp_table(oracle_lib):
    table = e2m1_table()
    for c in range(16):
        v = oracle_lib.e2m1(c)
        assert v == table[c], (c, v, table[c])
        assert math.copysign(1.0, v) == math.copysign(1.0, table[c]), c  # -0 for code 8


def test_e8m0_closed_form_exhaustive(oracle_lib):
    for e in range(255):
        assert oracle_lib.e8m0(e) == math.ldexp(1.0, e - 127), e
    assert math.isnan(oracle_lib.e8m0(255))


def test_fp16_decoder_matches_numpy_exhaustive(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle_lib.fp16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decoder(oracle_lib):
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 65536, size=4096).astype(np.uint16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32)
    got = np.array([oracle_lib.bf16(int(b)) for b in bits], dtype=np.float32)
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok].view(np.uint32), ref[ok].view(np.uint32))


def test_bf16_rounding_of_generator():
    # f32_to_bf16_bits must round to nearest even, checked on hand-made cases.
    cases = {
        np.float32(1.0): 0x3F80,
        np.float32(1.0) + np.float32(2.0 ** -8): 0x3F80,        # exact tie -> even
        np.float32(1.0) + np.float32(3 * 2.0 ** -8): 0x3F82,    # tie -> even (up)
        np.float32(1.0) + np.float32(2.0 ** -8 + 2.0 ** -20): 0x3F81,
        np.float32(-2.5): 0xC020,
    }
    for v, b in cases.items():
        assert int(W.f32_to_bf16_bits(np.array([v]))[0]) == b, (v, hex(b))


@pytest.mark.parametrize("n,k", [(16, 32), (32, 128), (48, 256)])
def test_mxfp4_layout_roundtrip_and_oracle_fetch(oracle_lib, n, k):
    rng = np.random.default_rng(n * 1000 + k)
    codes = rng.integers(0, 16, size=(n, k))
    scales = rng.integers(100, 140, size=(n, k // 32))
    cb, sb = mx_pack(codes, scales)
    assert cb.size == n * k // 2 and sb.size == n * k // 32
    c2, s2 = mx_unpack(cb, sb, n, k)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    table = e2m1_table()
    for _ in range(300):
        i, j = int(rng.integers(n)), int(rng.integers(k))
        want = table[codes[i, j]] * math.ldexp(1.0, int(scales[i, j // 32]) - 127)
        assert oracle_lib.mxfp4_weight(cb, sb, n, k, i, j) == want


def test_mxfp4_single_nibble_positions(oracle_lib):
    """Placing one non-zero code anywhere must light exactly that weight: this
    catches swapped nibbles, swapped row/column or a wrong tile stride."""
    n, k = 32, 64
    for (i, j) in [(0, 0), (0, 1), (1, 0), (15, 31), (16, 0), (3, 33), (31, 63), (17, 62)]:
        codes = np.zeros((n, k), dtype=np.int64)
        codes[i, j] = 7  # +6.0
        scales = np.full((n, k // 32), 127)
        cb, sb = mx_pack(codes, scales)
        dense = np.array([[oracle_lib.mxfp4_weight(cb, sb, n, k, a, b) for b in range(k)]
                          for a in range(n)])
        nz = np.argwhere(dense != 0)
        assert nz.tolist() == [[i, j]], (i, j, nz.tolist())
        assert dense[i, j] == 6.0


def test_oracle_decode_matrix_matches_numpy_unpacker(oracle_lib):
    wl = W.TINY
    packed = W.make_experts(wl)
    from helpers import mx_expert_dense
    for e in (0, 5):
        g, u, d = mx_expert_dense(wl, packed, e)
        gu = oracle_lib.decode_matrix(wl.fmt, wl.hidden, wl.inter, wl.experts, packed, e, 0)
        dn = oracle_lib.decode_matrix(wl.fmt, wl.hidden, wl.inter, wl.experts, packed, e, 1)
        assert np.array_equal(gu[:wl.inter], g) and np.array_equal(gu[wl.inter:], u)
        assert np.array_equal(dn, d)


def test_mxfp4_config_values_exact_in_bf16(oracle_lib):
    """Every (code, exponent) pair the configs use (exponents 120..126) is a
    bf16 value, so a bf16 dequantisation of these weights is exact."""
    for e in range(120, 127):
        for c in range(16):
            v = oracle_lib.e2m1(c) * oracle_lib.e8m0(e)
            f32 = np.float32(v)
            assert float(f32) == v
            bits = np.array([f32]).view(np.uint32)[0]
            assert bits & 0xFFFF == 0, (c, e)


def test_vq_layout_roundtrip(oracle_lib):
    rng = np.random.default_rng(7)
    n, k = 32, 512
    i13 = rng.integers(0, 8192, size=(n, k // 8))
    i8 = rng.integers(0, 256, size=(n, k // 8)).astype(np.uint8)
    gains = rng.uniform(0.5, 1.5, size=n).astype(np.float16)
    code12, plane, res, gain = vq_pack(i13, i8, gains)
    c, p, r, g = W.vq_matrix_regions(n, k)
    assert (code12.size, plane.size, res.size, gain.size) == (c, p, r, g)
    a13, a8 = vq_unpack(code12, plane, res, n, k)
    assert np.array_equal(a13, i13) and np.array_equal(a8, i8)
    pos = vq_positions(n, k)
    assert np.array_equal(np.sort(pos.reshape(-1)), np.arange(n * k // 8))


def _vq_layer_with(i13_fn, i8_fn, cb, rb, gains_fn, h=256, i=256, e=2, seed=0):
    """Packed VQ layer built with the numpy packer from index/gain functions."""
    rng = np.random.default_rng(seed)
    parts = [cb.astype(np.float16).view(np.uint8).reshape(-1),
             rb.astype(np.float16).view(np.uint8).reshape(-1)]
    for _ in range(e):
        for (n, k) in ((2 * i, h), (h, i)):
            i13 = i13_fn(rng, n, k)
            i8 = i8_fn(rng, n, k)
            g = gains_fn(rng, n)
            parts.extend(vq_pack(i13, i8.astype(np.uint8), g))
    return np.concatenate(parts)


def test_vq_zero_residual_equals_r13_only(oracle_lib):
    """With a zero residual book, weights are gain * Cb[i13] exactly: the
    13-bit stage is unchanged by the residual stage (Baekpica VQ card,
    "Recipe")."""
    rng = np.random.default_rng(3)
    cb = rng.standard_normal((8192, 8)).astype(np.float16)
    rb = np.zeros((256, 8), dtype=np.float16)
    packed = _vq_layer_with(lambda r, n, k: r.integers(0, 8192, size=(n, k // 8)),
                            lambda r, n, k: r.integers(0, 256, size=(n, k // 8)),
                            cb, rb, lambda r, n: r.uniform(0.5, 1.5, n).astype(np.float16))
    h = i = 256
    got = oracle_lib.decode_matrix(W.FMT_VQ13R8, h, i, 2, packed, 1, 0)
    # recover indices with the numpy unpacker and form gain * Cb[i13]
    base = W.VQ_BOOKS_BYTES + W.vq_expert_bytes(h, i)
    c, p, r, g = W.vq_matrix_regions(2 * i, h)
    i13, _ = vq_unpack(packed[base:base + c], packed[base + c:base + c + p],
                       packed[base + c + p:base + c + p + r], 2 * i, h)
    gain = packed[base + c + p + r:base + c + p + r + g].view(np.float16).astype(np.float64)
    want = gain[:, None] * cb.astype(np.float64)[i13].reshape(2 * i, h)
    assert np.array_equal(got, want)


def test_vq13_layer_is_the_13_bit_stage(oracle_lib):
    """A VQ13 layer (no residual stage) holding the 13-bit stage of a VQ13R8
    layer whose residual book is zero decodes to the same weights and gives
    the same layer output bit for bit (adding the residual stage leaves the
    13-bit stage's bytes unchanged: Baekpica VQ card, "Recipe").  The
    VQ13 buffer is the VQ13R8 one with the residual regions cut out."""
    rng = np.random.default_rng(4)
    cb = rng.standard_normal((8192, 8)).astype(np.float16)
    rb = np.zeros((256, 8), dtype=np.float16)
    h, i, e = 256, 256, 2
    packed = _vq_layer_with(lambda r, n, k: r.integers(0, 8192, size=(n, k // 8)),
                            lambda r, n, k: r.integers(0, 256, size=(n, k // 8)),
                            cb, rb, lambda r, n: r.uniform(0.5, 1.5, n).astype(np.float16),
                            h=h, i=i, e=e)
    p13 = W.vq13_from_vq13r8(packed, h, i, e)
    assert p13.size == W.packed_bytes(W.FMT_VQ13, h, i, e)
    for ex in range(e):
        for which in (0, 1):
            a = oracle_lib.decode_matrix(W.FMT_VQ13R8, h, i, e, packed, ex, which)
            b = oracle_lib.decode_matrix(W.FMT_VQ13, h, i, e, p13, ex, which)
            assert np.array_equal(a, b)
    wl = W.TINY_VQ13.replace(experts=e, tokens=5)
    x, wr = W.make_x(wl), W.make_router(wl)
    ra = oracle_lib.moe_forward(W.FMT_VQ13R8, h, i, e, 2, packed, x, wr)
    rb13 = oracle_lib.moe_forward(W.FMT_VQ13, h, i, e, 2, p13, x, wr)
    assert np.array_equal(ra["out"], rb13["out"])


def test_vq13_sizes():
    """13 bits per 8 weights plus an fp16 gain per row: 5,128,192 bytes per
    MiMo-shaped expert; the layer's book is the 128 KiB Cb alone."""
    assert W.vq_expert_bytes(4096, 2048, res=False) == 3 * 2048 * 4096 * 13 // 64 + 2 * (
        2 * 2048 + 4096) == 5128192
    assert W.packed_bytes(W.FMT_VQ13, 4096, 2048, 256) == 8192 * 16 + 256 * 5128192


def test_vq_unit_vector_books_closed_form(oracle_lib):
    """Cb[j] = ((j % 1024) + 1) * 2^-(j // 1024) * e_(j mod 8) and
    Rb[m] = -m/256 * e_((m+3) mod 8), all exact in fp16.  Then
    w[n][8v+d] = gain[n] * (Cb term if d == i13 % 8, minus i8/256 if
    d == (i8+3) % 8).  Indices span all 13 bits, so the plane bit matters."""
    def cb_val(j):
        return ((j % 1024) + 1) * 2.0 ** -(j // 1024)
    cb = np.zeros((8192, 8))
    for j in range(8192):
        cb[j, j % 8] = cb_val(j)
    assert np.array_equal(cb.astype(np.float16).astype(np.float64), cb)
    rb = np.zeros((256, 8))
    for m in range(256):
        rb[m, (m + 3) % 8] = -m / 256.0
    packed = _vq_layer_with(lambda r, n, k: r.integers(0, 8192, size=(n, k // 8)),
                            lambda r, n, k: r.integers(0, 256, size=(n, k // 8)),
                            cb, rb, lambda r, n: np.full(n, 0.5, dtype=np.float16))
    h = i = 256
    got = oracle_lib.decode_matrix(W.FMT_VQ13R8, h, i, 2, packed, 0, 1)   # down of expert 0
    base = W.VQ_BOOKS_BYTES + sum(W.vq_matrix_regions(2 * i, h))
    c, p, r, _ = W.vq_matrix_regions(h, i)
    i13, i8 = vq_unpack(packed[base:base + c], packed[base + c:base + c + p],
                        packed[base + c + p:base + c + p + r], h, i)
    assert i13.max() >= 4096
    want = np.zeros((h, i))
    for n in range(h):
        for v in range(i // 8):
            a, b = int(i13[n, v]), int(i8[n, v])
            want[n, 8 * v + a % 8] += cb_val(a)
            want[n, 8 * v + (b + 3) % 8] -= b / 256.0
    assert np.array_equal(got, 0.5 * want)


def test_generator_sizes_match_payload_formula():
    # MXFP4: 4.25 bit per weight, 3*I*H weights per expert.
    assert W.mxfp4_expert_bytes(4096, 2048) == 3 * 2048 * 4096 * 17 // 32 == 13369344
    assert W.packed_bytes(W.FMT_MXFP4, 4096, 2048, 256) == 3422552064
    assert W.mxfp4_expert_bytes(256, 128) * 8 == 417792
    # VQ R13+8: 21 bits per 8 weights plus an fp16 gain per row.
    assert W.vq_expert_bytes(4096, 2048) == 3 * 2048 * 4096 * 21 // 64 + 2 * (2 * 2048 + 4096)
    assert W.VQ_BOOKS_BYTES == 135168


def test_generated_codes_and_scales_distribution():
    wl = W.TINY
    packed = W.make_experts(wl)
    reg = W.mxfp4_expert_regions(wl.hidden, wl.inter)
    ex = packed.reshape(wl.experts, -1)
    for name in ("gu_scales", "dn_scales"):
        a, b = reg[name]
        s = ex[:, a:b]
        assert s.min() >= 120 and s.max() <= 126
    a, b = reg["gu_codes"]
    lo = ex[:, a:b] & 15
    counts = np.bincount(lo.reshape(-1), minlength=16)
    assert counts.min() > 0.8 * counts.mean()
    # determinism
    assert W.sha256(packed) == W.sha256(W.make_experts(wl))
