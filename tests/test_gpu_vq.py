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
    """All tokens on experts 0 and 1: 150 tokens per expert, a full 128-token
    pass of each (expert, slice) item and a second one of 22 tokens."""
    wl = W.TINY_VQ.replace(tokens=150, seed=21)
    wr = np.zeros((wl.experts, wl.hidden), dtype=np.float32)
    got, _, _ = _full_check(torch_dev, wl, PRE, wr=wr)
    assert got["counts"][:2].tolist() == [150, 150]


@pytest.mark.parametrize("t", [17, 32, 33, 48, 49, 64, 65, 80, 81, 96, 97, 112, 113, 128, 129])
def test_tiny_vq_grouped_tile_counts(torch_dev, t):
    """A zero router gives experts 0 and 1 all t tokens (t > 16: the grouped
    GEMM): each compiled token-tile count of a pass (2 to 8 tiles of 16, a lone
    tile run as two) at its edges, the switch from two K steps per LDS slot
    (up to 112 tokens) to one (113 and more), and a second pass."""
    wl = W.TINY_VQ.replace(tokens=t, seed=300 + t)
    wr = np.zeros((wl.experts, wl.hidden), dtype=np.float32)
    got, _, _ = _full_check(torch_dev, wl, PRE, wr=wr)
    assert got["counts"][:2].tolist() == [t, t]


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
    top-8, 2048 tokens): routing of every token bit for bit; outputs on at
    least 64 rows chosen so that every routed expert's codes meet some sampled
    token."""
    from test_gpu_parity import _sampled_check, covering_sample
    wl = W.VQ_PREFILL
    got, sample = _sampled_check(torch_dev, wl, PRE, lambda r: covering_sample(r["idx"], 64),
                                 packed=W.make_experts(wl))
    assert got["counts"].sum() == wl.tokens * wl.top_k and len(sample) >= 64
    assert set(np.unique(got["idx"][sample])) == set(np.nonzero(got["counts"])[0])


def test_mimo_vq_verify_t16(torch_dev):
    """The VQ13R8 16-token verify batch the benchmark times: the MiMo-shaped
    VQ13R8 layer, the skewed verify router and tokens, the AUTO path (the
    one-token-tile grouped GEMM over the active experts); every row."""
    from test_gpu_parity import _sampled_check
    wl = W.VERIFY.replace(fmt=W.FMT_VQ13R8, name="mimo_vq_verify_t16_skewed")
    got, _ = _sampled_check(torch_dev, wl, AUTO, list(range(16)),
                            packed=W.make_experts(W.VQ_PREFILL))
    assert got["path"] == PRE
    assert 40 <= int((got["counts"] > 0).sum()) <= 128


@pytest.mark.parametrize("t", [3, 8])
def test_mimo_vq_verify_widths(torch_dev, t):
    """The narrower verify widths of the benchmark's sweep (3 drafted tokens,
    and 8) on the MiMo-shaped VQ13R8 layer with the skewed router, AUTO path
    (the small-batch kernel over the active experts); every row."""
    from test_gpu_parity import _sampled_check
    wl = W.VERIFY.replace(fmt=W.FMT_VQ13R8, tokens=t, name=f"mimo_vq_verify_t{t}_skewed")
    got, _ = _sampled_check(torch_dev, wl, AUTO, list(range(t)),
                            packed=W.make_experts(W.VQ_PREFILL))
    assert got["path"] == PRE
    assert got["counts"].sum() == t * wl.top_k


@pytest.mark.parametrize("fmt", [W.FMT_VQ13R8, W.FMT_VQ13], ids=["vq13r8", "vq13"])
@pytest.mark.parametrize("t", [5, 16])
def test_vq_small_batch_chained_passes(torch_dev, fmt, t):
    """Small batches (2..16 tokens) at a shape where both GEMMs have a multiple
    of four 256-column super-steps (hidden 2048: 8, intermediate 1024: 4) and
    the active experts give every block two or more items, so each block's
    passes load their successors' first index streams; every row."""
    wl = W.TINY_VQ.replace(hidden=2048, inter=1024, experts=128, top_k=8, tokens=t, fmt=fmt,
                           seed=400 + t + 10 * fmt, name=f"vq_small_chain_{fmt}_{t}")
    got, _, _ = _full_check(torch_dev, wl, PRE)
    assert int((got["counts"] > 0).sum()) >= min(t * 8, 128) // 3
