"""The C ABI library loads, exports every entry point include/bqmoe.h
declares, and rejects bad arguments on the host before any device call.
CPU only: nothing here launches a kernel."""

import ctypes
import os
import re

import pytest

import bit_quantized_moe_gemv_amd as bq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bqmoe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bq.LIB_PATH):
        from bit_quantized_moe_gemv_amd import build
        build.build()
    return bq.load_library()


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert _header_functions() == sorted(bq.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _header_functions():
        assert hasattr(lib, name), name
    nm = os.popen(f"nm -D --defined-only {bq.LIB_PATH}").read()
    for name in _header_functions():
        assert re.search(rf"\bT {name}\b", nm), name


def test_status_strings(lib):
    assert bq.status_str(0) == "ok"
    for c in (bq.MOE_EINVAL, bq.MOE_EUNSUPPORTED, bq.MOE_EWORKSPACE, bq.MOE_EHIP):
        assert bq.status_str(c) and bq.status_str(c) != "unknown status"


def test_sizes_for_the_mimo_layer(lib):
    assert bq.packed_size(4096, 2048, 256, 8) == 3422552064
    assert bq.packed_size(256, 128, 8, 2) == 417792
    ws = bq.workspace_size(4096, 2048, 256, 8, 2048)
    r = 2048 * 8
    # per route: h (fp32), y (fp16 with one exponent byte per 4 or 16 columns),
    # the fp16 copy of h and its exponent
    per_route = 2048 * 4 + 4096 * 2 + 4096 // 4 + 2048 * 2 + 4
    assert ws >= r * per_route
    assert ws < r * per_route + 8 * 2**20


@pytest.mark.parametrize("bad", [
    dict(hidden=200), dict(hidden=0), dict(hidden=8448), dict(hidden=16384), dict(inter=96), dict(n_experts=0), dict(n_experts=300),
    dict(top_k=0), dict(top_k=9), dict(top_k=9, n_experts=8), dict(max_tokens=0),
    dict(fmt=7), dict(force_path=5),
])
def test_descriptor_validation(lib, bad):
    d = dict(hidden=256, inter=128, n_experts=8, top_k=2, max_tokens=16, fmt=1, force_path=0)
    d.update(bad)
    with pytest.raises(bq.MoeError) as ei:
        bq.packed_size(**d)
    assert ei.value.status == bq.MOE_EINVAL


def test_largest_hidden_accepted(lib):
    """hidden 8192 is the largest width every path takes (the small-batch
    router holds a token's row in 32 groups of 256 columns)."""
    assert bq.packed_size(8192, 128, 8, 2) == 3 * 128 * 8192 * 17 // 32 * 8
    assert bq.workspace_size(8192, 128, 8, 2, 16) > 0


def test_top_k_larger_than_experts_rejected(lib):
    with pytest.raises(bq.MoeError):
        bq.packed_size(256, 128, 4, 8)


def test_create_and_forward_validation_without_device(lib):
    d = bq.moe_layer_desc(256, 128, 8, 2, 16, 1, 0)
    ws = bq.workspace_size(256, 128, 8, 2, 16)
    h = ctypes.c_void_p(0)
    fake = 0x7F0000000000  # never dereferenced: validation fails or no launch happens
    assert lib.moe_layer_create(ctypes.byref(d), None, ws, ctypes.byref(h)) == bq.MOE_EWORKSPACE
    assert lib.moe_layer_create(ctypes.byref(d), fake + 16, ws, ctypes.byref(h)) == bq.MOE_EWORKSPACE
    assert lib.moe_layer_create(ctypes.byref(d), fake, ws - 1, ctypes.byref(h)) == bq.MOE_EWORKSPACE
    assert lib.moe_layer_create(ctypes.byref(d), fake, ws, None) == bq.MOE_EINVAL
    assert lib.moe_layer_create(ctypes.byref(d), fake, ws, ctypes.byref(h)) == bq.MOE_OK
    try:
        fw = lib.moe_layer_forward
        a = fake
        # T out of range, null and misaligned pointers: rejected before any launch
        assert fw(h, a, 0, a, a, a, None) == bq.MOE_EINVAL
        assert fw(h, a, 17, a, a, a, None) == bq.MOE_EINVAL
        assert fw(h, None, 1, a, a, a, None) == bq.MOE_EINVAL
        assert fw(h, a + 2, 1, a, a, a, None) == bq.MOE_EINVAL
        assert fw(h, a, 1, a + 4, a, a, None) == bq.MOE_EINVAL
        assert fw(h, a, 1, a, a + 8, a, None) == bq.MOE_EINVAL
        assert fw(h, a, 1, a, a, None, None) == bq.MOE_EINVAL
        assert fw(None, a, 1, a, a, a, None) == bq.MOE_EINVAL
        # no forward yet: routing and last_path report EINVAL
        assert lib.moe_layer_routing(h, None, None, None, None, None, None, None) == bq.MOE_EINVAL
        assert lib.moe_layer_last_path(h) == bq.MOE_EINVAL
    finally:
        lib.moe_layer_destroy(h)
    lib.moe_layer_destroy(None)


def test_forced_decode_rejects_large_batches(lib):
    d = bq.moe_layer_desc(256, 128, 8, 2, 64, 1, bq.MOE_PATH_DECODE)
    ws = bq.workspace_size(256, 128, 8, 2, 64, 1, bq.MOE_PATH_DECODE)
    h = ctypes.c_void_p(0)
    fake = 0x7F0000000000
    assert lib.moe_layer_create(ctypes.byref(d), fake, ws, ctypes.byref(h)) == bq.MOE_OK
    try:
        assert lib.moe_layer_forward(h, fake, 17, fake, fake, fake, None) == bq.MOE_EINVAL
    finally:
        lib.moe_layer_destroy(h)


def test_vq_descriptor_sizes_and_paths(lib):
    """VQ13R8 layers: packed size = books + experts; intermediate widths must be
    multiples of 256; forcing the decode path on a shape the batch-1 VQ
    kernels do not cover is reported as unsupported."""
    import workloads as W
    for h, i, e in ((256, 256, 8), (4096, 2048, 256)):
        assert bq.packed_size(h, i, e, 2, fmt=bq.MOE_FMT_VQ13R8) == \
            W.packed_bytes(W.FMT_VQ13R8, h, i, e)
    with pytest.raises(bq.MoeError) as ei:
        bq.packed_size(256, 128, 8, 2, fmt=bq.MOE_FMT_VQ13R8)
    assert ei.value.status == bq.MOE_EINVAL
    # batch-1 decode kernels exist for hidden/256 in {1, 2, 4, 8, 16} and
    # inter in {256, 512, 1024, 2048}; other shapes cannot be forced to decode
    for h, i in ((256, 256), (512, 2048), (4096, 2048), (4096, 256)):
        bq.workspace_size(h, i, 8, 2, 16, bq.MOE_FMT_VQ13R8, bq.MOE_PATH_DECODE)
    for h, i in ((768, 512), (8192, 2048), (4096, 4096), (1024, 768)):
        with pytest.raises(bq.MoeError) as ei:
            bq.workspace_size(h, i, 8, 2, 16, bq.MOE_FMT_VQ13R8, bq.MOE_PATH_DECODE)
        assert ei.value.status == bq.MOE_EUNSUPPORTED
    # the VQ workspace adds the fp16 copy of x, its row exponents and the
    # largest |h| of each 64-column piece of every route's h row
    mx = bq.workspace_size(4096, 2048, 256, 8, 2048, bq.MOE_FMT_MXFP4)
    vq = bq.workspace_size(4096, 2048, 256, 8, 2048, bq.MOE_FMT_VQ13R8)
    extra = 2048 * 4096 * 2 + 2048 * 4 + 2048 * 8 * (2048 // 64) * 4
    assert extra <= vq - mx < extra + 3 * 256


def test_routing_field_validated(lib):
    """routing 0 (softmax) and 1 (sigmoid) are accepted; other values are not."""
    for r in (bq.MOE_ROUTE_SOFTMAX, bq.MOE_ROUTE_SIGMOID):
        assert bq.workspace_size(256, 128, 8, 2, 16, routing=r) > 0
    for r in (-1, 2, 7):
        with pytest.raises(bq.MoeError) as ei:
            bq.workspace_size(256, 128, 8, 2, 16, routing=r)
        assert ei.value.status == bq.MOE_EINVAL


def test_vq13_descriptor_sizes(lib):
    import workloads as W
    for h, i, e in ((256, 256, 8), (4096, 2048, 256), (768, 512, 4)):
        assert bq.packed_size(h, i, e, 2, fmt=bq.MOE_FMT_VQ13) == W.packed_bytes(W.FMT_VQ13, h, i, e)
    with pytest.raises(bq.MoeError) as ei:
        bq.packed_size(256, 128, 8, 2, fmt=bq.MOE_FMT_VQ13)
    assert ei.value.status == bq.MOE_EINVAL
    # batch-1 decode kernels cover VQ13 like VQ13R8
    bq.workspace_size(4096, 2048, 256, 8, 1, bq.MOE_FMT_VQ13, bq.MOE_PATH_DECODE)
    with pytest.raises(bq.MoeError) as ei:
        bq.packed_size(256, 256, 8, 2, fmt=4)
    assert ei.value.status == bq.MOE_EINVAL


def test_binding_rejects_mismatched_tensors(lib):
    """MoeLayer.forward checks dtype, shape, contiguity, byte size and device
    of every tensor before the C call (the kernels would otherwise index past
    a too-small or differently laid out buffer).  A CPU workspace suffices:
    every case here is refused before anything reaches the library, so the
    checks run on a handle-less instance with a CPU workspace."""
    import torch
    layer = bq.MoeLayer.__new__(bq.MoeLayer)
    layer.hidden, layer.n_experts, layer.max_tokens = 256, 8, 16
    layer._packed_bytes = bq.packed_size(256, 128, 8, 2)
    layer.workspace = torch.empty(16, dtype=torch.uint8)
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    wr = torch.zeros((8, 256), dtype=torch.float32)
    pk = torch.zeros(layer.packed_bytes, dtype=torch.uint8)
    out = torch.zeros((4, 256), dtype=torch.float32)
    bad = [
        dict(x=x.float()), dict(x=torch.zeros((4, 512), dtype=torch.bfloat16)),
        dict(x=torch.zeros((17, 256), dtype=torch.bfloat16)),
        dict(x=torch.zeros((256, 4), dtype=torch.bfloat16).t()),
        dict(router_w=wr.half()), dict(router_w=torch.zeros((7, 256))),
        dict(router_w=torch.zeros((256, 8)).t()),
        dict(packed=pk[:-1]), dict(packed=pk.view(torch.int8)),
        dict(out=out.double()), dict(out=torch.zeros((4, 128))),
        dict(out=torch.zeros((256, 4)).t()),
    ]
    for kw in bad:
        args = dict(x=x, router_w=wr, packed=pk, out=out)
        args.update(kw)
        with pytest.raises(ValueError):
            layer._check_args(args["x"], args["router_w"], args["packed"], args["out"])
    layer._check_args(x, wr, pk, out)  # the matching set passes


def test_noalloc_validates_before_any_device_call(lib):
    """moe_forward_noalloc checks its arguments and the workspace size before
    it touches a device: with no GPU here, reaching the device would return
    MOE_EHIP, so these codes show the order.  97 MiMo-shaped tokens need more
    than the 16 MiB array."""
    desc = bq.moe_layer_desc(4096, 2048, 256, 8, 112, 1, 0, 0)
    p = 1 << 20  # aligned, never dereferenced
    f = lib.moe_forward_noalloc
    assert bq.workspace_size(4096, 2048, 256, 8, 96) <= bq.MOE_NOALLOC_SCRATCH_BYTES
    assert bq.workspace_size(4096, 2048, 256, 8, 97) > bq.MOE_NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(desc), p, 97, p, p, p, None) == bq.MOE_EWORKSPACE
    assert f(ctypes.byref(desc), p, 0, p, p, p, None) == bq.MOE_EINVAL
    assert f(ctypes.byref(desc), p, 113, p, p, p, None) == bq.MOE_EINVAL
    assert f(ctypes.byref(desc), p + 8, 4, p, p, p, None) == bq.MOE_EINVAL
    assert f(None, p, 4, p, p, p, None) == bq.MOE_EINVAL
    bad = bq.moe_layer_desc(4096, 2048, 256, 9, 112, 1, 0, 0)
    assert f(ctypes.byref(bad), p, 4, p, p, p, None) == bq.MOE_EINVAL
    forced = bq.moe_layer_desc(4096, 2048, 256, 8, 112, 1, bq.MOE_PATH_DECODE, 0)
    assert f(ctypes.byref(forced), p, 17, p, p, p, None) == bq.MOE_EINVAL
