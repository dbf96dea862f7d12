"""GPU parity of the VQ13R8 large-batch kernels (every batch of two or more
tokens, and forced batches of one) against the CPU oracle on the same seeded inputs: routing bit for bit, the
output per token row within relative L2 2e-3 and max |error| 1e-2 * rms."""

import numpy as np
import pytest

import workloads as W
from test_gpu_parity import PRE, _full_check, _routing_exact, torch_dev  # noqa: F401
from helpers import check_output

pytestmark = pytest.mark.gpu

AUTO = 0


def test_tiny_vq_layer(torch_dev):
    got, _, _ = _full_check(torch_dev, W.TINY_VQ, PRE)
    assert got["counts"].sum() == W.TINY_VQ.tokens * W.TINY_VQ.top_k


@pytest.mark.parametrize("t", [2, 3, 7])
def test_tiny_vq_ragged_token_counts_auto_path(torch_dev, t):
    """Small batches of two or more tokens take the large-batch kernels."""
    from gpu_harness import Runner
    import oracle
    wl = W.TINY_VQ.replace(tokens=t, seed=200 + t)
    x, wr = W.make_x(wl), W.make_router(wl)
    run = Runner(wl, AUTO)
    got = run.run(x, wr)
    assert got["path"] == PRE
    _routing_exact(got, oracle.route(x, wr, wl.top_k), wl)
    ref = oracle.moe_forward(wl.fmt, wl.hidden, wl.inter, wl.experts, wl.top_k,
                             run.packed_host, x, wr)
    check_output(got["out"], ref["out"])


def test_tiny_vq_zero_router_multi_chunk(torch_dev):
    """All tokens on experts 0 and 1: 150 tokens per expert, three 64-token
    chunks spread over both chunk lanes of each (expert, slice) item."""
    wl = W.TINY_VQ.replace(tokens=150, seed=21)
    wr = np.zeros((wl.experts, wl.hidden), dtype=np.float32)
    got, _, _ = _full_check(torch_dev, wl, PRE, wr=wr)
    assert got["counts"][:2].tolist() == [150, 150]


def test_tiny_vq_zero_input(torch_dev):
    wl = W.TINY_VQ
    x = np.zeros((wl.tokens, wl.hidden), dtype=np.uint16)
    got, _, _ = _full_check(torch_dev, wl, PRE, x=x)
    assert np.all(got["out"] == 0)


def test_tiny_vq_ragged_medium(torch_dev):
    _full_check(torch_dev, W.TINY_VQ.replace(tokens=333, seed=22), PRE)


@pytest.mark.parametrize("scale", [64.0, 2.0 ** 40, 2.0 ** -60])
def test_tiny_vq_scaled_tokens(torch_dev, scale):
    """Rows far outside fp16's range (x up to ~2^42, h up to ~2^84, or tiny):
    the per-row power-of-two exponents keep the fp16 operands in range."""
    wl = W.TINY_VQ.replace(tokens=64, seed=23, scaled_tokens=6, token_scale=scale)
    _full_check(torch_dev, wl, PRE)


def test_tiny_vq_wide_shapes(torch_dev):
    """hidden 768 (three 256-column super-steps, odd) and intermediate 512;
    the down slices of 512 rows end in a half slice."""
    wl = W.TINY_VQ.replace(hidden=768, inter=512, tokens=40, seed=24, name="vq_wide")
    _full_check(torch_dev, wl, PRE)


def test_tiny_vq_determinism(torch_dev):
    from gpu_harness import Runner
    wl = W.TINY_VQ.replace(tokens=200, seed=25)
    x, wr = W.make_x(wl), W.make_router(wl)
    run = Runner(wl, PRE)
    assert np.array_equal(run.run(x, wr)["out"], run.run(x, wr)["out"])


def test_mimo_vq_prefill_2048(torch_dev):
    """The full VQ13R8 layer (hidden 4096, intermediate 2048, 256 experts,
    top-8, 2048 tokens) on sampled token rows."""
    from gpu_harness import Runner, log
    import oracle
    wl = W.VQ_PREFILL
    sample = [0, 1, 777, 1500, 2047]
    log(f"case {wl.name} T={wl.tokens} sample={sample}")
    x, wr = W.make_x(wl), W.make_router(wl)
    run = Runner(wl, PRE)
    got = run.run(x, wr)
    _routing_exact(got, oracle.route(x, wr, wl.top_k), wl)
    assert got["counts"].sum() == wl.tokens * wl.top_k
    ref = oracle.moe_forward(wl.fmt, wl.hidden, wl.inter, wl.experts, wl.top_k,
                             run.packed_host, x, wr, tokens=sample)
    l2, mx = check_output(got["out"][np.asarray(sample)], ref["out"])
    log(f"  worst sampled row: rel l2 {l2:.2e}, max/rms {mx:.2e}")
    assert np.all(np.isfinite(got["out"]))
