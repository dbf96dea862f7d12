"""GPU parity of VQ13 layers (the 13-bit stage alone, no residual book)
against the CPU oracle on the same seeded inputs: routing bit for bit, the
output per token row within relative L2 2e-3 and max |error| 1e-2 * rms."""

import numpy as np
import pytest

import workloads as W
from test_gpu_parity import DEC, PRE, _full_check, _routing_exact, torch_dev  # noqa: F401
from helpers import check_output

pytestmark = pytest.mark.gpu

AUTO = 0


@pytest.mark.parametrize("seed", [81, 82])
def test_vq13_decode_batch1(torch_dev, seed):
    _full_check(torch_dev, W.TINY_VQ13.replace(tokens=1, seed=seed, top_k=8), DEC)


@pytest.mark.parametrize("t", [1, 3, 16, 150])
def test_vq13_grouped_gemm(torch_dev, t):
    """The grouped-GEMM kernels: one-tile small batches (t <= 16, t = 1
    forced) and 64-token chunks."""
    _full_check(torch_dev, W.TINY_VQ13.replace(tokens=t, seed=90 + t), PRE)


def test_vq13_wide_shapes(torch_dev):
    wl = W.TINY_VQ13.replace(hidden=768, inter=512, tokens=40, seed=95, name="vq13_wide")
    _full_check(torch_dev, wl, PRE)
    _full_check(torch_dev, W.TINY_VQ13.replace(hidden=1024, inter=2048, tokens=1, seed=96,
                                               name="vq13_dec_wide"), DEC)


@pytest.mark.parametrize("scale", [2.0 ** 40, 2.0 ** -60])
def test_vq13_scaled_tokens(torch_dev, scale):
    wl = W.TINY_VQ13.replace(tokens=64, seed=97, scaled_tokens=6, token_scale=scale)
    _full_check(torch_dev, wl, PRE)
    _full_check(torch_dev, wl.replace(tokens=1, scaled_tokens=1, seed=98), DEC)


def test_vq13_auto_path_and_sigmoid(torch_dev):
    from gpu_harness import Runner
    wl = W.TINY_VQ13.replace(tokens=1, seed=99, routing=1)
    run = Runner(wl, AUTO)
    assert run.run(W.make_x(wl), W.make_router(wl))["path"] == DEC
    _full_check(torch_dev, wl, DEC)


def test_mimo_vq13_decode_batch1(torch_dev):
    """The MiMo-shaped VQ13 layer (256 experts of 5,128,192 bytes) at one
    token, in the launch configuration the benchmark times."""
    from gpu_harness import Runner, log
    import oracle
    wl = W.VQ13_DECODE
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
