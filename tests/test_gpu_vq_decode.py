"""GPU parity of the batch-1 VQ13R8 decode kernels against the CPU oracle on
the same seeded inputs: routing bit for bit, the output per token row within
relative L2 2e-3 and max |error| 1e-2 * rms."""

import numpy as np
import pytest

import workloads as W
from test_gpu_parity import DEC, PRE, _full_check, _routing_exact, torch_dev  # noqa: F401
from helpers import check_output

pytestmark = pytest.mark.gpu

AUTO = 0


@pytest.mark.parametrize("seed", [41, 42, 43])
def test_tiny_vq_decode(torch_dev, seed):
    _full_check(torch_dev, W.TINY_VQ.replace(tokens=1, seed=seed), DEC)


@pytest.mark.parametrize("h,i", [(512, 512), (1024, 1024), (2048, 2048), (4096, 256),
                                 (256, 2048)])
def test_vq_decode_shapes(torch_dev, h, i):
    """Every kernel instance: hidden/256 of 1 to 16 (the gate/up wave splits)
    and inter/256 of 1 to 8 (the down tiles per wave)."""
    wl = W.TINY_VQ.replace(hidden=h, inter=i, tokens=1, seed=h + i, name=f"vq_dec_{h}x{i}")
    _full_check(torch_dev, wl, DEC)


@pytest.mark.parametrize("k,e", [(1, 8), (3, 8), (5, 8), (8, 8), (8, 64)])
def test_vq_decode_top_k(torch_dev, k, e):
    """k below, at and above the four routes of one down phase; k = E."""
    wl = W.TINY_VQ.replace(top_k=k, experts=e, tokens=1, seed=60 + k + e,
                           name=f"vq_dec_k{k}_e{e}")
    got, _, _ = _full_check(torch_dev, wl, DEC)
    assert got["counts"].sum() == k


def test_vq_decode_zero_router(torch_dev):
    """All logits +0: experts 0..k-1 with equal weights."""
    wl = W.TINY_VQ.replace(tokens=1, top_k=4, seed=44)
    wr = np.zeros((wl.experts, wl.hidden), dtype=np.float32)
    got, _, _ = _full_check(torch_dev, wl, DEC, wr=wr)
    assert got["idx"][0].tolist() == [0, 1, 2, 3]
    assert np.all(got["w"] == np.float32(0.25))


def test_vq_decode_zero_input(torch_dev):
    wl = W.TINY_VQ.replace(tokens=1, seed=45)
    x = np.zeros((1, wl.hidden), dtype=np.uint16)
    got, _, _ = _full_check(torch_dev, wl, DEC, x=x)
    assert np.all(got["out"] == 0)


@pytest.mark.parametrize("scale", [2.0 ** 40, 2.0 ** -60])
def test_vq_decode_scaled_token(torch_dev, scale):
    """x far outside fp16's range (up to ~2^42, h up to ~2^84) or tiny: the
    per-row power-of-two exponents of x and h keep the fp16 operands exact."""
    wl = W.TINY_VQ.replace(tokens=1, seed=46, scaled_tokens=1, token_scale=scale)
    _full_check(torch_dev, wl, DEC)


def test_vq_auto_path_by_batch(torch_dev):
    """AUTO takes the decode kernels at one token and the grouped-GEMM kernels
    from two tokens on; both agree with the oracle."""
    from gpu_harness import Runner
    import oracle
    for t, path in ((1, DEC), (2, PRE)):
        wl = W.TINY_VQ.replace(tokens=t, seed=47)
        x, wr = W.make_x(wl), W.make_router(wl)
        run = Runner(wl, AUTO, max_tokens=16)
        got = run.run(x, wr)
        assert got["path"] == path
        _routing_exact(got, oracle.route(x, wr, wl.top_k), wl)
        ref = oracle.moe_forward(wl.fmt, wl.hidden, wl.inter, wl.experts, wl.top_k,
                                 run.packed_host, x, wr)
        check_output(got["out"], ref["out"])


def test_vq_forced_decode_rejects_two_tokens(torch_dev):
    import bit_quantized_moe_gemv_amd as bq
    from gpu_harness import Runner
    wl = W.TINY_VQ.replace(tokens=2, seed=48)
    run = Runner(wl, DEC)
    with pytest.raises(bq.MoeError) as ei:
        run.run(W.make_x(wl), W.make_router(wl))
    assert ei.value.status == bq.MOE_EINVAL


def test_vq_decode_determinism_and_replay(torch_dev):
    """Two forwards give identical bits, and replaying every stage of the
    decode path (router, gate/up, down) leaves the output unchanged."""
    from gpu_harness import Runner
    import bit_quantized_moe_gemv_amd as bq
    torch = torch_dev
    wl = W.TINY_VQ.replace(tokens=1, seed=49, top_k=8)
    x, wr = W.make_x(wl), W.make_router(wl)
    run = Runner(wl, DEC)
    ref = run.run(x, wr)["out"]
    assert np.array_equal(run.run(x, wr)["out"], ref)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    wd = torch.from_numpy(wr).cuda()
    out = torch.zeros((1, wl.hidden), dtype=torch.float32, device="cuda")
    run.layer.forward(xd, wd, run.packed, out=out)
    st = torch.cuda.current_stream().cuda_stream
    args = (int(xd.data_ptr()), int(wd.data_ptr()), int(run.packed.data_ptr()), 0, 1,
            int(out.data_ptr()), st)
    for stage in ("router", "gateup", "down"):
        assert run.layer.replay_stage_raw(stage, 3, *args) == bq.MOE_OK
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)


def test_mimo_vq_decode_batch1(torch_dev):
    """The full VQ13R8 layer (hidden 4096, intermediate 2048, 256 experts,
    top-8) at one token, in the launch configuration the benchmark times."""
    from gpu_harness import Runner, log
    import oracle
    wl = W.VQ_PREFILL.replace(tokens=1, name="mimo_vq_decode_t1")
    log(f"case {wl.name} T=1")
    x, wr = W.make_x(wl), W.make_router(wl)
    run = Runner(wl, AUTO)
    got = run.run(x, wr)
    assert got["path"] == DEC
    _routing_exact(got, oracle.route(x, wr, wl.top_k), wl)
    ref = oracle.moe_forward(wl.fmt, wl.hidden, wl.inter, wl.experts, wl.top_k,
                             run.packed_host, x, wr)
    l2, mx = check_output(got["out"], ref["out"])
    log(f"  rel l2 {l2:.2e}, max/rms {mx:.2e}")


def test_vq_decode_sigmoid_routing(torch_dev):
    for seed in (70, 71):
        _full_check(torch_dev, W.TINY_VQ.replace(tokens=1, seed=seed, top_k=8, routing=1), DEC)
    _full_check(torch_dev, W.TINY_VQ.replace(tokens=9, seed=72, routing=1), PRE)
