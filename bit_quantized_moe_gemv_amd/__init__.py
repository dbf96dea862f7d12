"""Python binding of libbqmoe.so, the gfx950 routed-expert MoE layer with
MXFP4 / VQ-coded experts.

This module only marshals arguments: every step of the layer runs in the HIP
kernels behind the C ABI declared in include/bqmoe.h.  PyTorch supplies the
device memory (tensor data pointers) and the stream; there is no CPU or
PyTorch fallback -- if the library is missing, loading fails loudly.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
# BQMOE_LIBRARY points the binding at another build of the same library
LIB_PATH = os.environ.get("BQMOE_LIBRARY") or os.path.join(_PKG, "libbqmoe.so")

MOE_OK = 0
MOE_EINVAL = -1
MOE_EUNSUPPORTED = -2
MOE_EWORKSPACE = -3
MOE_EHIP = -4

MOE_FMT_MXFP4 = 1
MOE_FMT_VQ13R8 = 2
MOE_FMT_VQ13 = 3

MOE_PATH_AUTO = 0
MOE_PATH_DECODE = 1
MOE_PATH_PREFILL = 2
MOE_ROUTE_SOFTMAX = 0
MOE_ROUTE_SIGMOID = 1
MOE_DECODE_MAX_TOKENS = 16

STAGES = ("router", "select", "permute", "gateup", "down", "combine")

EXPORTED_SYMBOLS = (
    "moe_packed_size",
    "moe_workspace_size",
    "moe_layer_create",
    "moe_layer_forward",
    "moe_layer_routing",
    "moe_layer_last_path",
    "moe_layer_set_profiling",
    "moe_layer_profile_read",
    "moe_layer_replay_stage",
    "moe_read_probe",
    "moe_forward_noalloc",
    "moe_layer_destroy",
    "moe_status_str",
)


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} ({status})")
        self.status = status


class moe_layer_desc(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32),
        ("format", ctypes.c_int32),
        ("force_path", ctypes.c_int32),
        ("routing", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libbqmoe.so (built in-tree by build.py).  Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python bit_quantized_moe_gemv_amd/build.py or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    D = ctypes.POINTER(moe_layer_desc)
    lib.moe_packed_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_packed_size.restype = ctypes.c_int
    lib.moe_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_workspace_size.restype = ctypes.c_int
    lib.moe_layer_create.argtypes = [D, P, ctypes.c_size_t, ctypes.POINTER(P)]
    lib.moe_layer_create.restype = ctypes.c_int
    lib.moe_layer_forward.argtypes = [P, P, ctypes.c_int32, P, P, P, P]
    lib.moe_layer_forward.restype = ctypes.c_int
    lib.moe_layer_routing.argtypes = [P, P, P, P, P, P, P, P]
    lib.moe_layer_routing.restype = ctypes.c_int
    lib.moe_layer_last_path.argtypes = [P]
    lib.moe_layer_last_path.restype = ctypes.c_int
    lib.moe_layer_destroy.argtypes = [P]
    lib.moe_layer_destroy.restype = None
    lib.moe_layer_set_profiling.argtypes = [P, ctypes.c_int32]
    lib.moe_layer_set_profiling.restype = ctypes.c_int
    lib.moe_layer_profile_read.argtypes = [P, ctypes.POINTER(ctypes.c_float), ctypes.c_int32]
    lib.moe_layer_profile_read.restype = ctypes.c_int
    lib.moe_layer_replay_stage.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P, P, P,
                                           ctypes.c_size_t, ctypes.c_int32, P, P]
    lib.moe_layer_replay_stage.restype = ctypes.c_int
    lib.moe_read_probe.argtypes = [P, ctypes.c_size_t, ctypes.c_size_t, ctypes.c_int32,
                                   ctypes.c_int32, P, P]
    lib.moe_read_probe.restype = ctypes.c_int
    lib.moe_forward_noalloc.argtypes = [D, P, ctypes.c_int32, P, P, P, P]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_status_str.argtypes = [ctypes.c_int]
    lib.moe_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().moe_status_str(status).decode()


def _desc(hidden, inter, n_experts, top_k, max_tokens, fmt, force_path,
          routing=MOE_ROUTE_SOFTMAX) -> moe_layer_desc:
    return moe_layer_desc(hidden, inter, n_experts, top_k, max_tokens, fmt, force_path, routing)


def packed_size(hidden, inter, n_experts, top_k, max_tokens=1, fmt=MOE_FMT_MXFP4,
                force_path=MOE_PATH_AUTO, routing=MOE_ROUTE_SOFTMAX) -> int:
    b = ctypes.c_size_t(0)
    rc = load_library().moe_packed_size(
        ctypes.byref(_desc(hidden, inter, n_experts, top_k, max_tokens, fmt, force_path, routing)),
        ctypes.byref(b))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_packed_size")
    return b.value


def workspace_size(hidden, inter, n_experts, top_k, max_tokens, fmt=MOE_FMT_MXFP4,
                   force_path=MOE_PATH_AUTO, routing=MOE_ROUTE_SOFTMAX) -> int:
    b = ctypes.c_size_t(0)
    rc = load_library().moe_workspace_size(
        ctypes.byref(_desc(hidden, inter, n_experts, top_k, max_tokens, fmt, force_path, routing)),
        ctypes.byref(b))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_workspace_size")
    return b.value


def read_probe(buf_ptr: int, nbytes: int, copy_stride: int, n_copies: int, reps: int,
               sink_ptr: int, stream_ptr: int) -> None:
    """Enqueue `reps` plain streaming reads of nbytes (moe_read_probe)."""
    rc = load_library().moe_read_probe(buf_ptr, nbytes, copy_stride, n_copies, reps, sink_ptr,
                                       ctypes.c_void_p(stream_ptr))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_read_probe")


MOE_NOALLOC_SCRATCH_BYTES = 16 << 20


def forward_noalloc_raw(desc: moe_layer_desc, x_ptr: int, T: int, router_ptr: int,
                        packed_ptr: int, out_ptr: int, stream_ptr: int) -> int:
    """moe_forward_noalloc at pointer level (no checks): the forward pass with
    the library's own per-GPU workspace array; returns the status code."""
    return load_library().moe_forward_noalloc(ctypes.byref(desc), x_ptr, T, router_ptr,
                                              packed_ptr, out_ptr, ctypes.c_void_p(stream_ptr))


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


@dataclass
class Routing:
    topk_idx: object
    topk_w: object
    counts: object
    offsets: object
    perm: object
    logits: object


class MoeLayer:
    """One routed-expert layer handle with a torch-allocated workspace.

    forward(x, router_w, packed, out=None) runs the whole layer on the
    current torch stream; x is a [T, hidden] bfloat16 CUDA tensor, router_w a
    [n_experts, hidden] float32 tensor, packed a uint8 tensor in the layer's
    packed format; the result is a [T, hidden] float32 tensor."""

    def __init__(self, hidden, inter, n_experts, top_k, max_tokens, fmt=MOE_FMT_MXFP4,
                 force_path=MOE_PATH_AUTO, device="cuda", routing=MOE_ROUTE_SOFTMAX):
        import torch

        self._lib = load_library()
        self.desc = _desc(hidden, inter, n_experts, top_k, max_tokens, fmt, force_path, routing)
        self.hidden, self.inter, self.n_experts, self.top_k = hidden, inter, n_experts, top_k
        self.max_tokens, self.fmt, self.force_path = max_tokens, fmt, force_path
        self.routing_mode = routing
        ws_bytes = workspace_size(hidden, inter, n_experts, top_k, max_tokens, fmt, force_path,
                                  routing)
        self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
        h = ctypes.c_void_p(0)
        rc = self._lib.moe_layer_create(ctypes.byref(self.desc), _ptr(self.workspace), ws_bytes,
                                        ctypes.byref(h))
        if rc != MOE_OK:
            raise MoeError(rc, "moe_layer_create")
        self._handle = h
        self._last_T = 0
        self._packed_bytes = packed_size(hidden, inter, n_experts, top_k, max_tokens, fmt,
                                         force_path, routing)

    @property
    def packed_bytes(self) -> int:
        return self._packed_bytes

    def _check_args(self, x, router_w, packed, out):
        """Dtype, layout, shape and device of the tensors handed to the C ABI:
        the kernels index them by the descriptor's sizes, so a mismatch here
        would become an out-of-bounds device access."""
        import torch

        def need(ok, msg):
            if not ok:
                raise ValueError(f"MoeLayer.forward: {msg}")

        need(x.dim() == 2 and x.shape[1] == self.hidden and 1 <= x.shape[0] <= self.max_tokens,
             f"x must be [T, {self.hidden}] with 1 <= T <= {self.max_tokens}, got {tuple(x.shape)}")
        T = int(x.shape[0])
        for name, t, dt, shape in (("x", x, torch.bfloat16, (T, self.hidden)),
                                   ("router_w", router_w, torch.float32,
                                    (self.n_experts, self.hidden)),
                                   ("out", out, torch.float32, (T, self.hidden))):
            need(t.dtype == dt, f"{name} must be {dt}, got {t.dtype}")
            need(tuple(t.shape) == shape, f"{name} must have shape {shape}, got {tuple(t.shape)}")
            need(t.is_contiguous(), f"{name} must be contiguous")
        need(packed.dtype == torch.uint8 and packed.is_contiguous(),
             "packed must be a contiguous uint8 tensor")
        need(packed.numel() >= self._packed_bytes,
             f"packed holds {packed.numel()} bytes, the layer needs {self._packed_bytes}")
        dev = self.workspace.device
        for name, t in (("x", x), ("router_w", router_w), ("packed", packed), ("out", out)):
            need(t.device == dev, f"{name} is on {t.device}, the layer's workspace on {dev}")

    def forward(self, x, router_w, packed, out=None, stream=None):
        import torch

        T = int(x.shape[0])
        if out is None:
            out = torch.empty((T, self.hidden), dtype=torch.float32, device=x.device)
        self._check_args(x, router_w, packed, out)
        if stream is None:
            stream = torch.cuda.current_stream(x.device)
        rc = self._lib.moe_layer_forward(self._handle, _ptr(x), T, _ptr(router_w), _ptr(packed),
                                         _ptr(out), ctypes.c_void_p(stream.cuda_stream))
        if rc != MOE_OK:
            raise MoeError(rc, "moe_layer_forward")
        self._last_T = T
        return out

    __call__ = forward

    def forward_raw(self, x_ptr: int, T: int, router_ptr: int, packed_ptr: int, out_ptr: int,
                    stream_ptr: int) -> int:
        """Pointer-level call (no checks); returns the status code."""
        return self._lib.moe_layer_forward(self._handle, x_ptr, T, router_ptr, packed_ptr,
                                           out_ptr, ctypes.c_void_p(stream_ptr))

    def replay_stage_raw(self, stage: str, reps: int, x_ptr: int, router_ptr: int,
                         packed_ptr: int, copy_stride: int, n_copies: int, out_ptr: int,
                         stream_ptr: int) -> int:
        """Re-run one stage (a name in STAGES) of the last forward reps times
        (moe_layer_replay_stage); returns the status code."""
        return self._lib.moe_layer_replay_stage(
            self._handle, STAGES.index(stage), reps, x_ptr, router_ptr, packed_ptr, copy_stride,
            n_copies, out_ptr, ctypes.c_void_p(stream_ptr))

    def routing(self, stream=None) -> Routing:
        import torch

        T, k, E = self._last_T, self.top_k, self.n_experts
        dev = self.workspace.device
        r = Routing(
            topk_idx=torch.empty((T, k), dtype=torch.int32, device=dev),
            topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
            counts=torch.empty(E, dtype=torch.int32, device=dev),
            offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
            perm=torch.empty(T * k, dtype=torch.int32, device=dev),
            logits=torch.empty((T, E), dtype=torch.float32, device=dev),
        )
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        rc = self._lib.moe_layer_routing(self._handle, _ptr(r.topk_idx), _ptr(r.topk_w),
                                         _ptr(r.counts), _ptr(r.offsets), _ptr(r.perm),
                                         _ptr(r.logits), ctypes.c_void_p(stream.cuda_stream))
        if rc != MOE_OK:
            raise MoeError(rc, "moe_layer_routing")
        return r

    def set_profiling(self, slots: int):
        """Record per-stage HIP event pairs for the next forwards (round robin
        over `slots`); 0 turns it off."""
        rc = self._lib.moe_layer_set_profiling(self._handle, slots)
        if rc != MOE_OK:
            raise MoeError(rc, "moe_layer_set_profiling")
        self._prof_slots = slots

    def profile_read(self):
        """Per-stage kernel milliseconds, a list (per slot) of dicts keyed by
        stage name; stages that did not run are absent."""
        n = getattr(self, "_prof_slots", 0)
        buf = (ctypes.c_float * (n * len(STAGES)))()
        rc = self._lib.moe_layer_profile_read(self._handle, buf, n)
        if rc != MOE_OK:
            raise MoeError(rc, "moe_layer_profile_read")
        out = []
        for s in range(n):
            row = {STAGES[i]: buf[s * len(STAGES) + i] for i in range(len(STAGES))
                   if buf[s * len(STAGES) + i] >= 0}
            out.append(row)
        return out

    def last_path(self) -> int:
        return self._lib.moe_layer_last_path(self._handle)

    def close(self):
        if getattr(self, "_handle", None) is not None and self._handle.value:
            self._lib.moe_layer_destroy(self._handle)
            self._handle = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
