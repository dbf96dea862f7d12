"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle
on the same seeded inputs.  Routing (logits, top-k indices, counts, offsets,
permutation) must match bit for bit; the output must satisfy, per token row,
relative L2 error <= 2e-3 and max |error| <= 1e-2 * rms of the row."""

import numpy as np
import pytest

import workloads as W
from helpers import check_output

pytestmark = pytest.mark.gpu

DEC = 1
PRE = 2


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_moe_gemv_amd as bq
    bq.load_library()
    return torch


def _routing_exact(got, ref, wl):
    assert np.array_equal(got["logits"].view(np.uint32), ref["logits"].view(np.uint32)), \
        "router logits differ bitwise"
    assert np.array_equal(got["idx"], ref["idx"])
    assert np.array_equal(got["counts"], ref["counts"])
    assert np.array_equal(got["offsets"], ref["offsets"])
    assert np.array_equal(got["perm"], ref["perm"])
    assert np.max(np.abs(got["w"] - ref["w"])) < 1e-5


def _full_check(torch_dev, wl, path, x=None, wr=None, packed=None, max_tokens=None):
    from gpu_harness import Runner, log
    import oracle
    log(f"case {wl.name} T={wl.tokens if x is None else x.shape[0]} path={path}")
    x = W.make_x(wl) if x is None else x
    wr = W.make_router(wl) if wr is None else wr
    run = Runner(wl, path, max_tokens=max_tokens or x.shape[0], packed=packed)
    got = run.run(x, wr)
    ref_route = oracle.route(x, wr, wl.top_k, wl.routing)
    ref = oracle.moe_forward(wl.fmt, wl.hidden, wl.inter, wl.experts, wl.top_k,
                             run.packed_host, x, wr, routing=wl.routing)
    assert got["path"] == path
    _routing_exact(got, ref_route, wl)
    l2, mx = check_output(got["out"], ref["out"])
    log(f"  worst row: rel l2 {l2:.2e}, max/rms {mx:.2e}")
    return got, ref, run


@pytest.mark.parametrize("path", [DEC, PRE], ids=["decode", "prefill"])
def test_tiny_layer(torch_dev, path):
    _full_check(torch_dev, W.TINY, path)


@pytest.mark.parametrize("path", [DEC, PRE], ids=["decode", "prefill"])
@pytest.mark.parametrize("t", [1, 3, 7])
def test_tiny_ragged_token_counts(torch_dev, path, t):
    wl = W.TINY.replace(tokens=t, seed=100 + t)
    _full_check(torch_dev, wl, path)


@pytest.mark.parametrize("path", [DEC, PRE], ids=["decode", "prefill"])
def test_zero_router_sends_all_tokens_to_first_experts(torch_dev, path):
    """All logits +0: every token picks experts 0..k-1, so two experts hold
    every route (exercises the multi-chunk loops of both paths)."""
    wl = W.TINY if path == DEC else W.TINY.replace(tokens=150, seed=11)
    wr = np.zeros((wl.experts, wl.hidden), dtype=np.float32)
    got, ref, _ = _full_check(torch_dev, wl, path, wr=wr)
    assert got["counts"][:wl.top_k].tolist() == [wl.tokens] * wl.top_k


@pytest.mark.parametrize("t", [1, 16, 17, 33, 48, 49, 64, 65, 80, 97, 112, 113, 128, 129, 241])
def test_prefill_expert_token_counts_around_two_chunks(torch_dev, t):
    """A zero router gives experts 0..k-1 all t tokens: every tile count of a
    128-token pass (1..8 tiles of 16 tokens), the ragged edges of several, and
    counts that take a second pass (129, 241).  The tile count is a
    compile-time parameter of the grouped GEMMs, and the waves whose 16 token
    rows lie past the pass's last token copy no B rows, so every count here
    runs a different kernel variant."""
    wl = W.TINY.replace(tokens=t, seed=200 + t)
    wr = np.zeros((wl.experts, wl.hidden), dtype=np.float32)
    got, _, _ = _full_check(torch_dev, wl, PRE, wr=wr)
    assert got["counts"][:wl.top_k].tolist() == [t] * wl.top_k


@pytest.mark.parametrize("hidden,inter", [(512, 512), (1024, 1024), (2048, 256), (8192, 128)])
@pytest.mark.parametrize("t", [1, 6])
def test_decode_kernel_shapes(torch_dev, hidden, inter, t):
    """The decode kernels are instantiated per hidden size (gate/up: 256-column
    super-steps per K slice, row groups per block) and per intermediate size
    (down: super-steps per K half); every hidden size from 512 to 8192 and every
    down instantiation runs here, at one token (routing inside the gate/up
    kernel) and at six."""
    wl = W.TINY.replace(tokens=t, hidden=hidden, inter=inter, experts=6, top_k=3,
                        seed=400 + hidden // 256 + t, name=f"dec_h{hidden}_i{inter}_t{t}")
    _full_check(torch_dev, wl, DEC)


@pytest.mark.parametrize("base,sizes,paths", [
    (W.TINY, (16, 17, 16, 1), (DEC, PRE, DEC, DEC)),
    (W.TINY_VQ, (1, 2, 1), (DEC, PRE, DEC)),
], ids=["mxfp4", "vq13r8"])
def test_auto_path_choice(torch_dev, base, sizes, paths):
    """With no forced path one handle serves every batch size up to its
    maximum: the decode kernels up to the threshold (16 tokens for MXFP4, one
    for VQ) and the grouped GEMM above it, switching back and forth between
    calls; both sides of the threshold agree with the oracle."""
    from gpu_harness import Runner, log
    import oracle
    run = Runner(base, 0, max_tokens=32)
    for t, want in zip(sizes, paths):
        wl = base.replace(tokens=t, seed=600 + t)
        log(f"case {base.name} AUTO T={t}")
        x, wr = W.make_x(wl), W.make_router(wl)
        got = run.run(x, wr)
        assert got["path"] == want, (t, got["path"])
        _routing_exact(got, oracle.route(x, wr, wl.top_k, wl.routing), wl)
        ref = oracle.moe_forward(wl.fmt, wl.hidden, wl.inter, wl.experts, wl.top_k,
                                 run.packed_host, x, wr, routing=wl.routing)
        check_output(got["out"], ref["out"])


@pytest.mark.parametrize("experts,k", [(8, 2), (256, 8)])
def test_single_token_tied_logits(torch_dev, experts, k):
    """Batch-1 decode with equal logits at the selection boundary: experts
    whose router rows are identical (and largest) tie, and the lowest indices
    must win, as must experts 0..k-1 when the router is all zero."""
    wl = W.TINY.replace(tokens=1, experts=experts, top_k=k, seed=300 + experts,
                        name=f"tiny_e{experts}_k{k}")
    x = W.make_x(wl)
    wr = W.make_router(wl)
    rng = np.random.default_rng(7)
    tied = np.sort(rng.choice(experts, size=k + 2, replace=False))
    wr[tied] = np.abs(wr[0]) * np.sign(W.bf16_bits_to_f32(x[0]).astype(np.float32)) * 3.0
    got, _, _ = _full_check(torch_dev, wl, DEC, x=x, wr=wr)
    assert sorted(got["idx"][0].tolist()) == tied[:k].tolist()
    got, _, _ = _full_check(torch_dev, wl, DEC, x=x, wr=np.zeros_like(wr))
    assert sorted(got["idx"][0].tolist()) == list(range(k))


@pytest.mark.parametrize("path", [DEC, PRE], ids=["decode", "prefill"])
def test_zero_input_gives_zero_output(torch_dev, path):
    wl = W.TINY
    x = np.zeros((wl.tokens, wl.hidden), dtype=np.uint16)
    got, _, _ = _full_check(torch_dev, wl, path, x=x)
    assert np.all(got["out"] == 0)


def test_prefill_ragged_medium(torch_dev):
    # several 64-token chunks per expert plus ragged tails
    wl = W.TINY.replace(tokens=333, seed=12)
    _full_check(torch_dev, wl, PRE)


def test_prefill_more_routes_than_one_permute_pass(torch_dev):
    """8300 tokens at k = 2: 16,600 routes, more than the 16,384 the
    permutation kernel holds in registers, so it takes its two-pass path."""
    wl = W.TINY.replace(tokens=8300, seed=17, name="tiny_t8300")
    _full_check(torch_dev, wl, PRE)


def test_prefill_scaled_tokens_tiny(torch_dev):
    wl = W.TINY.replace(tokens=64, seed=13, scaled_tokens=4, token_scale=64.0)
    _full_check(torch_dev, wl, PRE)


@pytest.mark.parametrize("path", [DEC, PRE], ids=["decode", "prefill"])
@pytest.mark.parametrize("lo,hi", [(110, 123), (100, 140)], ids=["span13", "span40"])
def test_wide_exponent_spans(torch_dev, path, lo, hi):
    """E8M0 exponents spread over 13 and over 40 binades in every row group.
    The prefill down GEMM scales each group's weights by its largest exponent
    into fp16: exact up to a span of 13, beyond that the lowest blocks lose
    bits far below the output tolerance."""
    wl = W.TINY.replace(tokens=16 if path == DEC else 48, seed=15, exp_lo=lo, exp_hi=hi)
    _full_check(torch_dev, wl, path)


@pytest.mark.parametrize("path", [DEC, PRE], ids=["decode", "prefill"])
def test_saturated_down_operands(torch_dev, path):
    """Every weight +6 (the largest E2M1 value) at one scale and every token
    0.9375: each h row is one value whose fp16 form lies just under 2^15, and
    every down product is the largest the grouped down GEMM can meet, so its
    fp32 sums reach 0.99 of the bound from which it scales the fp16 per-route
    outputs (I * 6 * 2^15 * 2^-ceil(log2(6 I))).  The outputs stay finite and
    match the oracle."""
    from helpers import e2m1_table, mx_pack_expert
    wl = W.TINY.replace(tokens=16 if path == DEC else 32, seed=17, name="tiny_saturated")
    h, i, e = wl.hidden, wl.inter, wl.experts
    six = int(np.nonzero(e2m1_table() == 6.0)[0][0])
    one = mx_pack_expert(wl, np.full((2 * i, h), six), np.full((2 * i, h // 32), 127),
                         np.full((h, i), six), np.full((h, i // 32), 127))
    packed = np.tile(one, e)
    x = np.full((wl.tokens, h), 0x3F70, dtype=np.uint16)  # bf16 0.9375
    got, ref, _ = _full_check(torch_dev, wl, path, x=x, packed=packed)
    g = 6.0 * h * 0.9375
    hv = g / (1.0 + np.exp(-g)) * g
    assert np.allclose(ref["out"], 6.0 * i * hv, rtol=1e-12)


def test_prefill_long_down_rows(torch_dev):
    """Intermediate 2176: 68 scale tiles per down row, more than one pass of
    the per-group exponent scan, and 17 K steps."""
    wl = W.TINY.replace(tokens=40, seed=16, inter=2176, experts=4, name="tiny_i2176")
    _full_check(torch_dev, wl, PRE)


def test_all_experts_active_k8(torch_dev):
    wl = W.TINY.replace(top_k=8, name="tiny_k8")
    for path in (DEC, PRE):
        _full_check(torch_dev, wl, path)


def test_determinism_bitwise(torch_dev):
    from gpu_harness import Runner
    for path, wl in ((DEC, W.TINY), (PRE, W.TINY.replace(tokens=200, seed=14))):
        x, wr = W.make_x(wl), W.make_router(wl)
        run = Runner(wl, path)
        a = run.run(x, wr)["out"]
        b = run.run(x, wr)["out"]
        assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# full MiMo shape (hidden 4096, intermediate 2048, 256 experts, top-8)
# ---------------------------------------------------------------------------

_LAYERS = {}


def _mimo_layer(seed):
    if seed not in _LAYERS:
        _LAYERS.clear()
        _LAYERS[seed] = W.make_experts(W.DECODE.replace(seed=seed))
    return _LAYERS[seed]


def covering_sample(idx, n_min, must=()):
    """Token rows in which every expert that some token routes to appears at
    least once (a greedy set cover over the routing idx [T, k]), together with
    the rows in `must`, topped up with evenly spaced rows to at least n_min
    rows (sorted)."""
    idx = np.asarray(idx)
    t, _ = idx.shape
    member = np.zeros((t, int(idx.max()) + 1), dtype=bool)
    member[np.arange(t)[:, None], idx] = True
    chosen = set(int(m) for m in must)
    uncovered = member.any(axis=0)
    for m in chosen:
        uncovered &= ~member[m]
    while uncovered.any():
        best = int(np.argmax((member & uncovered).sum(axis=1)))
        chosen.add(best)
        uncovered &= ~member[best]
    for m in np.linspace(0, t - 1, num=n_min).astype(int):
        if len(chosen) >= n_min:
            break
        chosen.add(int(m))
    return sorted(chosen)


def _sampled_check(torch_dev, wl, path, sample, packed=None):
    """Routing of every token bit for bit; the output on the rows `sample`
    names (a list, or a function of the oracle's routing that returns one)."""
    from gpu_harness import Runner, log
    import oracle
    log(f"case {wl.name} T={wl.tokens} path={path}")
    x, wr = W.make_x(wl), W.make_router(wl)
    packed = _mimo_layer(wl.seed) if packed is None else packed
    run = Runner(wl, path, packed=packed)
    got = run.run(x, wr)
    log("  gpu done; oracle routing")
    ref_route = oracle.route(x, wr, wl.top_k, wl.routing)
    if path != 0:
        assert got["path"] == path
    _routing_exact(got, ref_route, wl)
    if callable(sample):
        sample = sample(ref_route)
    log(f"  routing exact; oracle outputs of {len(sample)} rows: {list(sample)}")
    ref = oracle.moe_forward(wl.fmt, wl.hidden, wl.inter, wl.experts, wl.top_k, packed, x, wr,
                             tokens=sample, routing=wl.routing)
    l2, mx = check_output(got["out"][np.asarray(sample)], ref["out"])
    log(f"  worst sampled row: rel l2 {l2:.2e}, max/rms {mx:.2e}")
    assert np.all(np.isfinite(got["out"]))
    return got, sample


def test_mimo_decode_batch1(torch_dev):
    _sampled_check(torch_dev, W.DECODE, DEC, [0])


def test_mimo_verify_batch16_skewed(torch_dev):
    """Every row of the 16-token verify batch (skewed routing)."""
    got, _ = _sampled_check(torch_dev, W.VERIFY, DEC, list(range(16)))
    n_distinct = int((got["counts"] > 0).sum())
    assert 40 <= n_distinct <= 128


@pytest.mark.parametrize("t", [3, 8])
def test_mimo_verify_widths_decode_path(torch_dev, t):
    """Every row of the 3-token (MTP drafts) and 8-token (drafter block)
    verify widths of the sweep, on the decode kernels at the MiMo shape."""
    wl = W.VERIFY.replace(tokens=t, name=f"mimo_verify_t{t}_skewed")
    _sampled_check(torch_dev, wl, DEC, list(range(t)))


def test_mimo_prefill_2048(torch_dev):
    """The 2048-token prefill: routing of every token bit for bit; outputs on
    at least 64 rows chosen so that every routed expert's weights meet some
    sampled token, including all 20 tokens scaled by 64."""
    wl = W.PREFILL
    scaled = W.scaled_token_ids(wl)
    got, sample = _sampled_check(
        torch_dev, wl, PRE, lambda r: covering_sample(r["idx"], 64, must=scaled))
    assert got["counts"].sum() == wl.tokens * wl.top_k
    assert set(scaled.tolist()) <= set(sample) and len(sample) >= 64
    assert set(np.unique(got["idx"][sample])) == set(np.nonzero(got["counts"])[0])


def test_overflowing_logits_route_in_range(torch_dev):
    """Activations at the bf16 maximum with opposite signs in the two halves of
    the row drive every router partial sum to +inf or -inf, so every logit is
    NaN (inf - inf).  A NaN ranks below every number, so the selection takes
    the lowest expert indices, [0, k), on every path (batch-1 MXFP4 and VQ
    decode, grouped GEMM), and the kernels never see an index outside [0, E)."""
    from gpu_harness import Runner, log
    import oracle
    cases = [(W.TINY.replace(tokens=1, name="tiny_t1_nan"), DEC),
             (W.TINY.replace(tokens=1, experts=256, top_k=8, name="tiny_e256_t1_nan"), DEC),
             (W.TINY.replace(tokens=3, name="tiny_t3_nan"), DEC),
             (W.TINY.replace(tokens=20, name="tiny_t20_nan"), PRE),
             (W.TINY_VQ.replace(tokens=1, name="tiny_vq_t1_nan"), DEC)]
    for wl, path in cases:
        log(f"case {wl.name} path={path}")
        x = np.empty((wl.tokens, wl.hidden), dtype=np.uint16)
        x[:, :wl.hidden // 2] = 0x7F7F   # +3.39e38
        x[:, wl.hidden // 2:] = 0xFF7F   # -3.39e38
        wr = np.ones((wl.experts, wl.hidden), dtype=np.float32)
        run = Runner(wl, path)
        got = run.run(x, wr)
        ref = oracle.route(x, wr, wl.top_k, wl.routing)
        assert np.all(np.isnan(got["logits"])) and np.all(np.isnan(ref["logits"]))
        want = np.tile(np.arange(wl.top_k, dtype=np.int32), (wl.tokens, 1))
        assert np.array_equal(got["idx"], want) and np.array_equal(ref["idx"], want)
        for name in ("counts", "offsets", "perm"):
            assert np.array_equal(got[name], ref[name]), name


@pytest.mark.parametrize("path", [DEC, PRE], ids=["decode", "prefill"])
def test_replay_stage_reproduces_forward(torch_dev, path):
    """moe_layer_replay_stage re-runs a stage of the last forward: replaying
    every stage of the path, in order, leaves the output bit-identical."""
    from gpu_harness import Runner
    import bit_quantized_moe_gemv_amd as bq
    torch = torch_dev
    wl = W.TINY.replace(tokens=5 if path == DEC else 90, seed=31)
    x, wr = W.make_x(wl), W.make_router(wl)
    run = Runner(wl, path)
    ref = run.run(x, wr)["out"]
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.from_numpy(ref.astype(np.float32)).cuda()
    st = torch.cuda.current_stream().cuda_stream
    layer = run.layer
    wd = torch.from_numpy(wr).cuda()
    run.layer.forward(xd, wd, run.packed, out=out)
    stages = (("router", "gateup", "down") if path == DEC else
              ("router", "select", "permute", "gateup", "down", "combine"))
    args = (int(xd.data_ptr()), int(wd.data_ptr()), int(run.packed.data_ptr()), 0, 1,
            int(out.data_ptr()), st)
    for stage in stages:
        assert layer.replay_stage_raw(stage, 3, *args) == bq.MOE_OK
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)
    if path == DEC:
        assert layer.replay_stage_raw("combine", 1, *args) == bq.MOE_EINVAL


SIGMOID = 1


@pytest.mark.parametrize("path", [DEC, PRE], ids=["decode", "prefill"])
@pytest.mark.parametrize("t", [1, 5, 16])
def test_sigmoid_routing_tiny(torch_dev, path, t):
    """Sigmoid routing weights (same selection, weights sigma(l)/sum sigma)."""
    wl = W.TINY.replace(tokens=t, seed=300 + t, routing=SIGMOID)
    _full_check(torch_dev, wl, path)


def test_sigmoid_routing_prefill_large_batch(torch_dev):
    _full_check(torch_dev, W.TINY.replace(tokens=200, seed=310, routing=SIGMOID), PRE)


def test_sigmoid_routing_extreme_logits(torch_dev):
    """Router rows scaled so that logits reach about +-1e3: the weights stay
    finite and match the oracle (every sigma is 0 or 1 in fp32 there)."""
    wl = W.TINY.replace(tokens=16, seed=311, routing=SIGMOID, router_std=20.0)
    for path in (DEC, PRE):
        got, _, _ = _full_check(torch_dev, wl, path)
        assert np.all(np.isfinite(got["w"]))


def test_mimo_decode_batch1_sigmoid(torch_dev):
    _sampled_check(torch_dev, W.DECODE.replace(routing=SIGMOID), DEC, [0])


def test_handles_on_concurrent_streams(torch_dev):
    """Handles share no state: four layers (batch-1 decode, 16-token decode,
    grouped MXFP4, grouped VQ13R8), each with its own workspace, run
    interleaved on two streams of default priority and give, bit for bit, what
    each gives alone on the default stream."""
    import bit_quantized_moe_gemv_amd as bq
    torch = torch_dev
    cases = [(W.TINY.replace(tokens=1, name="t1"), DEC), (W.TINY, DEC),
             (W.TINY.replace(tokens=200, seed=18), PRE), (W.TINY_VQ, PRE)]
    runs = []
    for wl, path in cases:
        x = torch.from_numpy(W.make_x(wl).view(np.int16)).cuda().view(torch.bfloat16)
        wr = torch.from_numpy(W.make_router(wl)).cuda()
        pk = torch.from_numpy(W.make_experts(wl)).cuda()
        layer = bq.MoeLayer(wl.hidden, wl.inter, wl.experts, wl.top_k, wl.tokens, wl.fmt, path)
        alone = layer.forward(x, wr, pk).clone()
        runs.append((layer, x, wr, pk, alone))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rep in range(3):  # a handle stays on one stream (calls sharing a handle serialize)
        for i, (layer, x, wr, pk, _) in enumerate(runs):
            s = streams[i % 2]
            with torch.cuda.stream(s):
                outs.append((i, layer.forward(x, wr, pk, stream=s)))
    torch.cuda.synchronize()
    for i, out in outs:
        assert torch.equal(out, runs[i][4]), f"case {i} differs on a concurrent stream"
    for layer, *_ in runs:
        layer.close()


def test_forward_in_a_captured_graph(torch_dev):
    """A forward makes no host syncs, allocations or memsets, so it can be
    captured into a graph: every replay (with eager forwards and
    synchronisations in between, and after the input is overwritten in
    place) matches the eager result bit for bit."""
    import bit_quantized_moe_gemv_amd as bq
    torch = torch_dev
    cases = [(W.TINY.replace(tokens=1, name="t1"), DEC), (W.TINY, DEC),
             (W.TINY.replace(tokens=200, seed=19), PRE), (W.TINY_VQ, PRE)]
    for wl, path in cases:
        x = torch.from_numpy(W.make_x(wl).view(np.int16)).cuda().view(torch.bfloat16)
        x2 = torch.from_numpy(W.make_x(wl.replace(seed=wl.seed + 50)).view(np.int16)).cuda() \
            .view(torch.bfloat16)
        wr = torch.from_numpy(W.make_router(wl)).cuda()
        pk = torch.from_numpy(W.make_experts(wl)).cuda()
        layer = bq.MoeLayer(wl.hidden, wl.inter, wl.experts, wl.top_k, wl.tokens, wl.fmt, path)
        ref1 = layer.forward(x, wr, pk).clone()
        ref2 = layer.forward(x2, wr, pk).clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            layer.forward(x, wr, pk, stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        xin = x.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            out = layer.forward(xin, wr, pk)
        for rep in range(3):
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref1), f"{wl.name}: replay {rep} differs"
            layer.forward(x2, wr, pk)  # eager work between replays
            torch.cuda.synchronize()
        xin.copy_(x2)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref2), f"{wl.name}: replay after the input changed differs"
        del g
        layer.close()
