"""moe_forward_noalloc (the forward pass on the library's own per-GPU workspace
array, for callers that cannot allocate) against moe_layer_forward through the
C ABI on the same inputs: two calls in a row, the second with fewer tokens, on
every path (batch-1 and small-batch MXFP4 decode, the grouped GEMMs, VQ13R8
batch-1 decode) at tiny and MiMo shapes.  Both run the same kernels, so the
outputs must agree bit for bit; a few rows of every output are also checked
against the oracle."""

import numpy as np
import pytest

import workloads as W
from helpers import check_output

pytestmark = pytest.mark.gpu

AUTO, DEC, PRE = 0, 1, 2


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_moe_gemv_amd as bq
    bq.load_library()
    return torch


def _inputs(torch, wl, tokens, packed):
    x = W.make_x(wl, tokens=tokens)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    wr = W.make_router(wl)
    return x, wr, xd, torch.from_numpy(wr).cuda()


def _pair(torch, wl, sizes, packed_host, oracle_rows=None):
    """Runs moe_forward_noalloc for each T in sizes (in order, one after the
    other on one stream), then moe_layer_forward on a fresh handle per T, and
    compares the outputs bit for bit."""
    import bit_quantized_moe_gemv_amd as bq
    from gpu_harness import log
    pk = torch.from_numpy(packed_host).cuda()
    st = torch.cuda.current_stream()
    desc = bq.moe_layer_desc(wl.hidden, wl.inter, wl.experts, wl.top_k, max(sizes), wl.fmt, AUTO,
                             wl.routing)
    runs = []
    for t in sizes:
        x, wr, xd, wd = _inputs(torch, wl.replace(seed=wl.seed + t), t, packed_host)
        out = torch.full((t, wl.hidden), float("nan"), dtype=torch.float32, device="cuda")
        rc = bq.forward_noalloc_raw(desc, xd.data_ptr(), t, wd.data_ptr(), pk.data_ptr(),
                                    out.data_ptr(), st.cuda_stream)
        assert rc == bq.MOE_OK, bq.status_str(rc)
        runs.append((t, x, wr, xd, wd, out))
    torch.cuda.synchronize()
    for t, x, wr, xd, wd, out in runs:
        log(f"case {wl.name} T={t}: no-alloc vs handle")
        layer = bq.MoeLayer(wl.hidden, wl.inter, wl.experts, wl.top_k, t, wl.fmt, AUTO,
                            routing=wl.routing)
        ref = layer.forward(xd, wd, pk)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{wl.name} T={t}: outputs differ"
        if oracle_rows is not None:
            import oracle
            rows = [r for r in oracle_rows if r < t]
            want = oracle.moe_forward(wl.fmt, wl.hidden, wl.inter, wl.experts, wl.top_k,
                                      packed_host, x, wr, tokens=rows, routing=wl.routing)
            check_output(out.cpu().numpy()[rows], want["out"])
        layer.close()


@pytest.mark.parametrize("wl,sizes", [
    (W.TINY, (16, 5)),                  # small-batch decode, then a smaller batch
    (W.TINY, (40, 1)),                  # grouped GEMM, then batch-1 decode
    (W.TINY.replace(routing=1), (23, 17)),
    (W.TINY_VQ, (9, 1)),                # VQ grouped GEMM, then VQ batch-1 decode
], ids=["mxfp4_16_5", "mxfp4_40_1", "mxfp4_sigmoid_23_17", "vq13r8_9_1"])
def test_noalloc_matches_forward_tiny(torch_dev, wl, sizes):
    _pair(torch_dev, wl, sizes, W.make_experts(wl), oracle_rows=range(4))


def test_noalloc_matches_forward_mimo(torch_dev):
    """The MiMo-shaped MXFP4 layer: the 16-token verify batch, then one token."""
    wl = W.VERIFY
    _pair(torch_dev, wl, (16, 1), W.make_experts(wl), oracle_rows=[0])
