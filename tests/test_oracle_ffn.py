"""Pins of the oracle's expert feed-forward and whole-layer output (CPU)."""

import numpy as np
import pytest

import workloads as W
from helpers import (dense_ffn, expert_dense, mx_pack, mx_unpack, silu_np, check_output)


def _xf(x):
    return W.bf16_bits_to_f32(x).astype(np.float64)


def _dense_layer(oracle_lib, wl, packed, x, wr):
    """Whole layer with numpy: numpy-unpacked dense experts, matmuls, and the
    oracle's routing (routing itself is pinned in test_oracle_routing)."""
    r = oracle_lib.route(x, wr, wl.top_k)
    xf = _xf(x)
    out = np.zeros((wl.tokens, wl.hidden))
    for e in range(wl.experts):
        g, u, d = expert_dense(wl, packed, e)
        y = dense_ffn(g, u, d, xf)
        for t in range(wl.tokens):
            for s in range(wl.top_k):
                if r["idx"][t, s] == e:
                    out[t] += r["w"][t, s] * y[t]
    # slot order matters for bitwise equality only; compare within 1e-12
    return out, r


@pytest.mark.parametrize("wl", [W.TINY, W.TINY_VQ], ids=["mxfp4", "vq"])
def test_oracle_matches_dense_numpy_layer(oracle_lib, wl):
    x = W.make_x(wl)
    wr = W.make_router(wl)
    packed = W.make_experts(wl)
    got = oracle_lib.workload_forward(wl, packed, x, wr)
    want, r = _dense_layer(oracle_lib, wl, packed, x, wr)
    assert np.array_equal(got["idx"], r["idx"])
    assert np.max(np.abs(got["out"] - want)) <= 1e-12 * np.max(np.abs(want))


def test_identical_experts_reduce_to_one_dense_mlp(oracle_lib):
    """If every expert holds the same weights, the routing weights sum to one
    and the layer is a single SwiGLU MLP, whatever the router does."""
    wl = W.TINY
    packed = W.make_experts(wl).reshape(wl.experts, -1)
    packed[:] = packed[3]
    packed = packed.reshape(-1)
    x = W.make_x(wl)
    wr = W.make_router(wl)
    got = oracle_lib.workload_forward(wl, packed, x, wr)["out"]
    g, u, d = expert_dense(wl, packed, 0)
    want = dense_ffn(g, u, d, _xf(x))
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


def test_zero_codes_give_exact_zero(oracle_lib):
    wl = W.TINY
    packed = W.make_experts(wl)
    reg = W.mxfp4_expert_regions(wl.hidden, wl.inter)
    ex = packed.reshape(wl.experts, -1)
    for name in ("gu_codes", "dn_codes"):
        a, b = reg[name]
        ex[:, a:b] = 0
    out = oracle_lib.workload_forward(wl, ex.reshape(-1), W.make_x(wl), W.make_router(wl))["out"]
    assert np.all(out == 0)


def test_zero_input_gives_zero_and_uniform_routing(oracle_lib):
    wl = W.TINY
    x = np.zeros((wl.tokens, wl.hidden), dtype=np.uint16)
    r = oracle_lib.workload_forward(wl, W.make_experts(wl), x, W.make_router(wl))
    assert np.all(r["out"] == 0)
    assert np.all(r["idx"] == np.arange(wl.top_k)) and np.all(r["w"] == 1.0 / wl.top_k)


def test_interm_div_rescaling_is_invariant(oracle_lib):
    """The EXL3 card's layer-47 workaround (benthecarman card, "Bitrate")
    scales up_proj by 1/128 and restores the factor before the down
    projection, folded into the weights.  In MXFP4 that is: every up-row
    exponent minus 7 and every down exponent plus 7.  With wide accumulation
    the output must not change at all."""
    wl = W.TINY
    x, wr = W.make_x(wl), W.make_router(wl)
    packed = W.make_experts(wl)
    base = oracle_lib.workload_forward(wl, packed, x, wr)["out"]
    h, i = wl.hidden, wl.inter
    reg = W.mxfp4_expert_regions(h, i)
    ex = packed.reshape(wl.experts, -1).copy()
    for e in range(wl.experts):
        a, b = reg["gu_codes"]
        sa, sb = reg["gu_scales"]
        codes, scales = mx_unpack(ex[e, a:b], ex[e, sa:sb], 2 * i, h)
        scales[i:] -= 7                       # up rows
        _, nsb = mx_pack(codes, scales)
        ex[e, sa:sb] = nsb
        da, db = reg["dn_scales"]
        ex[e, da:db] += 7
    got = oracle_lib.workload_forward(wl, ex.reshape(-1), x, wr)["out"]
    assert np.array_equal(got, base)


def test_all_experts_active_is_a_dense_softmax_mixture(oracle_lib):
    wl = W.TINY.replace(top_k=8, name="tiny_k8")
    x, wr, packed = W.make_x(wl), W.make_router(wl), W.make_experts(wl)
    got = oracle_lib.workload_forward(wl, packed, x, wr)["out"]
    l = oracle_lib.router_logits(x, wr).astype(np.float64)
    p = np.exp(l - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    want = np.zeros_like(got)
    for e in range(wl.experts):
        g, u, d = expert_dense(wl, packed, e)
        want += p[:, e:e + 1] * dense_ffn(g, u, d, _xf(x))
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


def test_silu_is_stable_for_large_arguments(oracle_lib):
    # A token scaled so far that g is huge must not produce inf/nan.
    wl = W.TINY.replace(scaled_tokens=4, token_scale=2.0 ** 40)
    r = oracle_lib.workload_forward(wl, W.make_experts(wl), W.make_x(wl), W.make_router(wl))
    assert np.all(np.isfinite(r["out"]))
    g = np.array([-1e300, -800.0, -1.0, 0.0, 1.0, 800.0, 1e300])
    assert np.all(np.isfinite(silu_np(g)))


def test_prefill_scaled_tokens_overflow_fp16(oracle_lib):
    """The prefill workload multiplies 1% of tokens by 64 so that SwiGLU
    intermediates exceed fp16's 65504, as the pages report for layer 47
    (TrevorJS card, "Recipe"; benthecarman card, "Bitrate").  Checked on the
    full hidden/intermediate widths with 8 experts of the same distribution."""
    wl = W.PREFILL.replace(experts=8, top_k=2, tokens=64, scaled_tokens=4)
    x, packed = W.make_x(wl), W.make_experts(wl)
    scaled = W.scaled_token_ids(wl)
    plain = [t for t in range(wl.tokens) if t not in set(scaled.tolist())][:1]
    h_scaled, _ = oracle_lib.expert_ffn(wl.fmt, wl.hidden, wl.inter, wl.experts, packed, 0,
                                        x[scaled[0]])
    h_plain, _ = oracle_lib.expert_ffn(wl.fmt, wl.hidden, wl.inter, wl.experts, packed, 0,
                                       x[plain[0]])
    assert np.abs(h_scaled).max() > 65504.0
    assert np.abs(h_plain).max() < 65504.0


def test_tolerance_helper_rejects_planted_errors():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((4, 256))
    check_output(ref + 1e-6 * rng.standard_normal(ref.shape), ref)
    bad = ref.copy()
    bad[2, 7] += 0.05 * np.sqrt((ref[2] ** 2).mean())
    with pytest.raises(AssertionError):
        check_output(bad, ref)
    bad = ref * (1 + 3e-3)
    with pytest.raises(AssertionError):
        check_output(bad, ref)
    with pytest.raises(AssertionError):
        check_output(np.where(ref > 2, np.nan, ref), ref)
