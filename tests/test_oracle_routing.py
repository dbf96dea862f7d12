"""Pins of the oracle's router, top-k selection and route grouping (CPU)."""

import numpy as np
import pytest

import workloads as W


def _bf16(vals):
    return W.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_router_fma_inside_a_partial(oracle_lib):
    """Within one partial sum each step is a fused multiply-add.  Columns 0 and
    1 both belong to partial 0.  x = (1, 1 + 2^-7), W = (-(1 + 2^-7 + 2^-23),
    1 + 2^-23): after column 0 the partial is -(1 + 2^-7 + 2^-23); the exact
    product at column 1 is 1 + 2^-7 + 2^-23 + 2^-30, so a fused step leaves
    2^-30 (a separate multiply would round the product and leave 0)."""
    h = 256
    x = np.zeros((1, h), dtype=np.float32)
    wr = np.zeros((1, h), dtype=np.float32)
    x[0, 0], x[0, 1] = 1.0, 1.0 + 2.0 ** -7
    wr[0, 0] = -(1.0 + 2.0 ** -7 + 2.0 ** -23)
    wr[0, 1] = 1.0 + 2.0 ** -23
    got = oracle_lib.router_logits(_bf16(x), wr)
    assert got[0, 0] == np.float32(2.0 ** -30)


def test_router_pairwise_tree_of_partials(oracle_lib):
    """Partials 0..3 (columns 0, 4, 8, 12) hold 1, 2^24, 1, -2^24.  The tree
    adds (1 + 2^24) -> 2^24 (ties to even) and (1 - 2^24) exactly, giving 1.
    A left-to-right sum would give 0 and the exact sum is 2."""
    h = 256
    x = np.zeros((1, h), dtype=np.float32)
    wr = np.zeros((1, h), dtype=np.float32)
    for col, val in ((0, 1.0), (4, 2.0 ** 24), (8, 1.0), (12, -2.0 ** 24)):
        x[0, col] = 1.0
        wr[0, col] = val
    got = oracle_lib.router_logits(_bf16(x), wr)
    assert got[0, 0] == np.float32(1.0)


def test_router_partial_assignment_interleaved_by_four(oracle_lib):
    """Columns 4c..4c+3 (mod 256) belong to partial c: put 2^24 in column 256
    (partial 0) and 1 in columns 1 and 257 (partial 0 too): the chain
    1 -> 1 + 2^24 -> ... stays in one partial.  Compare with placing the small
    terms in partial 1: the tree then gives a different, hand-derived value."""
    h = 512
    x = np.ones((1, h), dtype=np.float32)
    # case A: all three terms in partial 0, order by column: col 1 (1.0), col 256 (2^24), col 257 (1.0)
    wa = np.zeros((1, h), dtype=np.float32)
    wa[0, 1], wa[0, 256], wa[0, 257] = 1.0, 2.0 ** 24, 1.0
    # chain: 1 ; 1 + 2^24 -> 2^24 ; 2^24 + 1 -> 2^24
    assert oracle_lib.router_logits(_bf16(x), wa)[0, 0] == np.float32(2.0 ** 24)
    # case B: columns 4 and 260 are partial 1, column 256 is partial 0:
    wb = np.zeros((1, h), dtype=np.float32)
    wb[0, 4], wb[0, 256], wb[0, 260] = 1.0, 2.0 ** 24, 1.0
    # p0 = 2^24, p1 = 2 ; tree: 2^24 + 2 exactly representable
    assert oracle_lib.router_logits(_bf16(x), wb)[0, 0] == np.float32(2.0 ** 24 + 2)


def test_router_one_hot_and_zero(oracle_lib):
    rng = np.random.default_rng(1)
    h, e = 512, 16
    wr = rng.standard_normal((e, h)).astype(np.float32)
    for col in (0, 3, 255, 256, 511):
        x = np.zeros((1, h), dtype=np.float32)
        x[0, col] = 1.0
        got = oracle_lib.router_logits(_bf16(x), wr)
        assert np.array_equal(got[0], wr[:, col])
    z = oracle_lib.router_logits(np.zeros((2, h), dtype=np.uint16), wr)
    assert np.all(z == 0) and not np.any(np.signbit(z))


def test_router_power_of_two_scaling_is_exact(oracle_lib):
    wl = W.TINY
    x = W.make_x(wl)
    wr = W.make_router(wl)
    base = oracle_lib.router_logits(x, wr)
    xf = W.bf16_bits_to_f32(x)
    for s in (2.0 ** -3, 4.0, 64.0):
        xs = W.f32_to_bf16_bits(xf * np.float32(s))
        got = oracle_lib.router_logits(xs, wr)
        assert np.array_equal(got, base * np.float32(s))


def test_router_within_fp32_error_bound_of_f64(oracle_lib):
    """|l32 - l_exact| <= (H/64 + 6) * 2^-24 * sum|x*W| (a chain of H/64
    fused steps, then six tree levels); l_exact is the float64 sum, whose own
    error is far below this bound."""
    wl = W.DECODE.replace(tokens=8)
    x = W.make_x(wl)
    wr = W.make_router(wl)
    l32 = oracle_lib.router_logits(x, wr).astype(np.float64)
    l64 = oracle_lib.router_logits_f64(x, wr)
    xa = np.abs(W.bf16_bits_to_f32(x).astype(np.float64))
    mag = xa @ np.abs(wr.astype(np.float64)).T
    bound = (wl.hidden / 64 + 6) * 2.0 ** -24 * mag * 1.01
    assert np.all(np.abs(l32 - l64) <= bound)
    assert np.max(np.abs(l32 - l64)) > 0  # the orders do differ somewhere


def _brute_force_topk(l, k):
    e = l.shape[0]
    sel = []
    for a in range(e):
        beats = sum(1 for b in range(e) if (l[b] > l[a]) or (l[b] == l[a] and b < a))
        if beats < k:
            sel.append((beats, a))
    return [a for _, a in sorted(sel)]


def test_topk_against_brute_force_and_numpy(oracle_lib):
    rng = np.random.default_rng(5)
    for e, k in ((8, 2), (16, 8), (256, 8), (8, 8)):
        l = rng.standard_normal((20, e)).astype(np.float32)
        l[:, ::3] = np.round(l[:, ::3])  # plenty of exact ties
        idx, w = oracle_lib.topk(l, k)
        for t in range(l.shape[0]):
            assert idx[t].tolist() == _brute_force_topk(l[t], k)
            order = np.lexsort((np.arange(e), -l[t].astype(np.float64)))[:k]
            assert idx[t].tolist() == order.tolist()
        assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)


def test_topk_ties_signed_zero_and_duplicates(oracle_lib):
    l = np.array([[0.0, -0.0, 0.0, 1.0, 1.0, -1.0]], dtype=np.float32)
    idx, w = oracle_lib.topk(l, 4)
    assert idx[0].tolist() == [3, 4, 0, 1]
    # all-zero logits (x = 0) pick experts 0..k-1 with weight exactly 1/k
    idx, w = oracle_lib.topk(np.zeros((3, 16), dtype=np.float32), 8)
    assert np.all(idx == np.arange(8)) and np.all(w == 1.0 / 8)


def test_duplicated_router_rows_tie_to_lower_index(oracle_lib):
    wl = W.TINY
    wr = W.make_router(wl)
    wr[6] = wr[1]
    x = W.make_x(wl)
    l = oracle_lib.router_logits(x, wr)
    assert np.array_equal(l[:, 1], l[:, 6])
    idx, _ = oracle_lib.topk(l, wl.top_k)
    for t in range(wl.tokens):
        if 6 in idx[t]:
            assert 1 in idx[t] and list(idx[t]).index(1) < list(idx[t]).index(6)


def test_softmax_closed_form_two_values(oracle_lib):
    l = np.array([[3.0, 1.0, -5.0]], dtype=np.float32)
    idx, w = oracle_lib.topk(l, 2)
    assert idx[0].tolist() == [0, 1]
    assert w[0, 0] == pytest.approx(1.0 / (1.0 + np.exp(-2.0)), rel=1e-15)
    assert w[0, 1] == pytest.approx(1.0 / (1.0 + np.exp(2.0)), rel=1e-15)


def test_permutation_against_sorted_and_invariants(oracle_lib):
    rng = np.random.default_rng(9)
    for t, e, k in ((16, 8, 2), (300, 256, 8), (1, 256, 8), (64, 16, 16)):
        idx = np.stack([rng.permutation(e)[:k] for _ in range(t)]).astype(np.int32)
        counts, offsets, perm, inv = oracle_lib.permute(idx, e)
        assert counts.sum() == t * k  # k routes for every token (8 at the MiMo shape)
        assert np.array_equal(counts, np.bincount(idx.reshape(-1), minlength=e))
        assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
        routes = sorted(range(t * k), key=lambda r: (idx.reshape(-1)[r], r // k))
        assert perm.tolist() == routes
        assert np.array_equal(inv[perm], np.arange(t * k))
        assert counts.max() <= t


def test_workload_routing_invariants(oracle_lib):
    for wl in (W.TINY, W.VERIFY.replace(tokens=64)):
        x = W.make_x(wl)
        wr = W.make_router(wl)
        r = oracle_lib.route(x, wr, wl.top_k)
        idx = r["idx"]
        assert all(len(set(row)) == wl.top_k for row in idx.tolist())
        assert r["counts"].sum() == wl.tokens * wl.top_k
        assert np.all(idx >= 0) and np.all(idx < wl.experts)


def test_skewed_verify_routing_concentrates_on_hot_experts(oracle_lib):
    """The verify workload's 32 hot experts receive about half of all routes
    (checked on 1024 tokens of the same distribution)."""
    wl = W.VERIFY.replace(tokens=1024)
    x = W.make_x(wl)
    wr = W.make_router(wl)
    idx, _ = oracle_lib.topk(oracle_lib.router_logits(x, wr), wl.top_k)
    hot = set(W.hot_expert_ids(wl).tolist())
    frac = np.isin(idx, list(hot)).mean()
    assert 0.45 < frac < 0.55, frac


# --- sigmoid routing: same selection, weights sigma(l_s) / sum_j sigma(l_j)
# over the selected logits (TrevorJS card, "Architecture notes").

def test_sigmoid_routing_selects_like_softmax_and_sums_to_one(oracle_lib):
    rng = np.random.default_rng(21)
    l = rng.normal(0.0, 3.0, size=(40, 256)).astype(np.float32)
    i_soft, _ = oracle_lib.topk(l, 8, oracle_lib.ROUTE_SOFTMAX)
    i_sig, w_sig = oracle_lib.topk(l, 8, oracle_lib.ROUTE_SIGMOID)
    assert np.array_equal(i_soft, i_sig)  # sigma is increasing
    assert np.allclose(w_sig.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(w_sig, axis=1) <= 0)  # slot order = weight order


def test_sigmoid_routing_symmetric_pair_is_sigma(oracle_lib):
    """Two selected logits a and -a: sigma(a) + sigma(-a) = 1, so the first
    weight is sigma(a) = (1 + tanh(a/2)) / 2 (checked with tanh)."""
    for a in (0.25, 1.0, 3.5, 12.0):
        l = np.array([[a, -a, -40.0]], dtype=np.float32)
        idx, w = oracle_lib.topk(l, 2, oracle_lib.ROUTE_SIGMOID)
        assert idx[0].tolist() == [0, 1]
        assert w[0, 0] == pytest.approx((1.0 + np.tanh(a / 2.0)) / 2.0, rel=1e-14)
        assert w[0, 1] == pytest.approx((1.0 - np.tanh(a / 2.0)) / 2.0, rel=1e-12)


def test_sigmoid_routing_limits(oracle_lib):
    """Far below zero sigma(l) = e^l (1 - e^l + ...), so the weights approach
    the softmax over the same logits; far above zero every sigma is 1 to
    within e^-l, so the weights approach 1/k.  Zero logits give exactly 1/k."""
    rng = np.random.default_rng(22)
    base = rng.normal(0.0, 1.0, size=(8, 64)).astype(np.float32)
    _, w_soft = oracle_lib.topk(base - 60.0, 8, oracle_lib.ROUTE_SOFTMAX)
    _, w_low = oracle_lib.topk(base - 60.0, 8, oracle_lib.ROUTE_SIGMOID)
    # e^-60 ~ 1e-26 is far below double rounding: agreement to rounding
    assert np.max(np.abs(w_low - w_soft) / w_soft) < 1e-13
    _, w_high = oracle_lib.topk(base + 60.0, 8, oracle_lib.ROUTE_SIGMOID)
    assert np.max(np.abs(w_high - 1.0 / 8.0)) < 1e-15
    _, w_zero = oracle_lib.topk(np.zeros((3, 16), dtype=np.float32), 4,
                                oracle_lib.ROUTE_SIGMOID)
    assert np.all(w_zero == 0.25)


def test_sigmoid_routing_differs_from_softmax_in_between(oracle_lib):
    """Near zero the two weightings differ: logits (1, 0) give softmax
    e/(e+1) ~ 0.731 but sigmoid weights sigma(1)/(sigma(1)+1/2) ~ 0.594."""
    l = np.array([[1.0, 0.0]], dtype=np.float32)
    _, w_soft = oracle_lib.topk(l, 2, oracle_lib.ROUTE_SOFTMAX)
    _, w_sig = oracle_lib.topk(l, 2, oracle_lib.ROUTE_SIGMOID)
    s1 = (1.0 + np.tanh(0.5)) / 2.0
    assert w_soft[0, 0] == pytest.approx(np.e / (np.e + 1.0), rel=1e-14)
    assert w_sig[0, 0] == pytest.approx(s1 / (s1 + 0.5), rel=1e-14)
