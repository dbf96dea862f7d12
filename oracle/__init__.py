"""ctypes binding of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.  It
shares no code with the GPU path.  Arrays are numpy; nothing here touches a
GPU.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

FMT_MXFP4 = 1
FMT_VQ13R8 = 2
FMT_VQ13 = 3


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fp contraction)."""
    if force or not os.path.exists(LIB_PATH):
        cmd = ["gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-shared", "-fPIC", "-Wall", "-Wextra", "-o", LIB_PATH + ".tmp", SRC_PATH, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        lib.oracle_e2m1.restype = ctypes.c_double
        lib.oracle_e2m1.argtypes = [_INT]
        lib.oracle_e8m0.restype = ctypes.c_double
        lib.oracle_e8m0.argtypes = [_INT]
        lib.oracle_fp16.restype = ctypes.c_double
        lib.oracle_fp16.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16.restype = ctypes.c_float
        lib.oracle_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_num_threads.restype = _INT
        lib.oracle_num_threads.argtypes = []
        lib.oracle_mxfp4_weight.restype = ctypes.c_double
        lib.oracle_mxfp4_weight.argtypes = [_P, _P, _I64, _I64, _I64, _I64]
        lib.oracle_vq_weight.restype = ctypes.c_double
        lib.oracle_vq_weight.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64]
        lib.oracle_decode_matrix.restype = _INT
        lib.oracle_decode_matrix.argtypes = [_INT, _I64, _I64, _I64, _P, _I64, _INT, _P]
        lib.oracle_router_logits.restype = _INT
        lib.oracle_router_logits.argtypes = [_P, _P, _I64, _I64, _I64, _P]
        lib.oracle_router_logits_f64.restype = _INT
        lib.oracle_router_logits_f64.argtypes = [_P, _P, _I64, _I64, _I64, _P]
        lib.oracle_topk.restype = _INT
        lib.oracle_topk.argtypes = [_P, _I64, _I64, _I64, _INT, _P, _P]
        lib.oracle_permute.restype = _INT
        lib.oracle_permute.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P, _P]
        lib.oracle_expert_ffn.restype = _INT
        lib.oracle_expert_ffn.argtypes = [_INT, _I64, _I64, _I64, _P, _I64, _P, _P, _P]
        lib.oracle_moe_forward.restype = _INT
        lib.oracle_moe_forward.argtypes = [_INT, _I64, _I64, _I64, _I64, _INT, _P, _P, _P, _I64,
                                           _P, _I64, _P, _P, _P, _P]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def num_threads() -> int:
    return _load().oracle_num_threads()


def e2m1(code: int) -> float:
    return _load().oracle_e2m1(code)


def e8m0(e: int) -> float:
    return _load().oracle_e8m0(e)


def fp16(bits: int) -> float:
    return _load().oracle_fp16(bits)


def bf16(bits: int) -> float:
    return _load().oracle_bf16(bits)


def mxfp4_weight(codes: np.ndarray, scales: np.ndarray, n_rows: int, k_cols: int, n: int, k: int) -> float:
    return _load().oracle_mxfp4_weight(_ptr(codes), _ptr(scales), n_rows, k_cols, n, k)


def decode_matrix(fmt: int, hidden: int, inter: int, experts: int, packed: np.ndarray,
                  expert: int, which: int) -> np.ndarray:
    """Dense float64 matrix of one expert: which=0 gate/up [2I, H], which=1 down [H, I]."""
    shape = (2 * inter, hidden) if which == 0 else (hidden, inter)
    out = np.empty(shape, dtype=np.float64)
    _check(_load().oracle_decode_matrix(fmt, hidden, inter, experts, _ptr(packed), expert, which,
                                        _ptr(out)), "decode_matrix")
    return out


def router_logits(x: np.ndarray, wr: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    wr = np.ascontiguousarray(wr, dtype=np.float32)
    t, h = x.shape
    e = wr.shape[0]
    out = np.empty((t, e), dtype=np.float32)
    _check(_load().oracle_router_logits(_ptr(x), _ptr(wr), t, h, e, _ptr(out)), "router_logits")
    return out


def router_logits_f64(x: np.ndarray, wr: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    wr = np.ascontiguousarray(wr, dtype=np.float32)
    t, h = x.shape
    e = wr.shape[0]
    out = np.empty((t, e), dtype=np.float64)
    _check(_load().oracle_router_logits_f64(_ptr(x), _ptr(wr), t, h, e, _ptr(out)), "router_f64")
    return out


ROUTE_SOFTMAX = 0
ROUTE_SIGMOID = 1


def topk(logits: np.ndarray, k: int, routing: int = ROUTE_SOFTMAX) -> tuple[np.ndarray, np.ndarray]:
    """Top-k experts per token and their weights (softmax, or sigmoid routing)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    t, e = logits.shape
    idx = np.empty((t, k), dtype=np.int32)
    w = np.empty((t, k), dtype=np.float64)
    _check(_load().oracle_topk(_ptr(logits), t, e, k, routing, _ptr(idx), _ptr(w)), "topk")
    return idx, w


def permute(idx: np.ndarray, experts: int):
    """Returns counts [E], offsets [E+1], perm [R], inv [R] (int32)."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    t, k = idx.shape
    counts = np.empty(experts, dtype=np.int32)
    offsets = np.empty(experts + 1, dtype=np.int32)
    perm = np.empty(t * k, dtype=np.int32)
    inv = np.empty(t * k, dtype=np.int32)
    _check(_load().oracle_permute(_ptr(idx), t, k, experts, _ptr(counts), _ptr(offsets),
                                  _ptr(perm), _ptr(inv)), "permute")
    return counts, offsets, perm, inv


def route(x: np.ndarray, wr: np.ndarray, k: int, routing: int = ROUTE_SOFTMAX):
    """Logits, top-k and grouping for all tokens: dict of numpy arrays."""
    logits = router_logits(x, wr)
    idx, w = topk(logits, k, routing)
    counts, offsets, perm, inv = permute(idx, wr.shape[0])
    return dict(logits=logits, idx=idx, w=w, counts=counts, offsets=offsets, perm=perm, inv=inv)


def expert_ffn(fmt: int, hidden: int, inter: int, experts: int, packed: np.ndarray,
               expert: int, x_row: np.ndarray):
    x_row = np.ascontiguousarray(x_row, dtype=np.uint16)
    h = np.empty(inter, dtype=np.float64)
    y = np.empty(hidden, dtype=np.float64)
    _check(_load().oracle_expert_ffn(fmt, hidden, inter, experts, _ptr(packed), expert,
                                     _ptr(x_row), _ptr(h), _ptr(y)), "expert_ffn")
    return h, y


def moe_forward(fmt: int, hidden: int, inter: int, experts: int, top_k: int,
                packed: np.ndarray, x: np.ndarray, wr: np.ndarray, tokens=None,
                routing: int = ROUTE_SOFTMAX):
    """Layer output for the listed tokens (all when None).

    Returns dict(out [n,H] float64, idx [n,k] int32, w [n,k] float64,
    logits [n,E] float32, tokens [n] int64)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    wr = np.ascontiguousarray(wr, dtype=np.float32)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    t = x.shape[0]
    if tokens is None:
        tok = np.arange(t, dtype=np.int64)
    else:
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    n = tok.shape[0]
    out = np.empty((n, hidden), dtype=np.float64)
    idx = np.empty((n, top_k), dtype=np.int32)
    w = np.empty((n, top_k), dtype=np.float64)
    logits = np.empty((n, experts), dtype=np.float32)
    _check(_load().oracle_moe_forward(fmt, hidden, inter, experts, top_k, routing, _ptr(packed), _ptr(x),
                                      _ptr(wr), t, _ptr(tok), n, _ptr(out), _ptr(idx), _ptr(w),
                                      _ptr(logits)), "moe_forward")
    return dict(out=out, idx=idx, w=w, logits=logits, tokens=tok)


def workload_forward(wl, packed, x, wr, tokens=None):
    """moe_forward with the shapes of a workloads.Workload."""
    return moe_forward(wl.fmt, wl.hidden, wl.inter, wl.experts, wl.top_k, packed, x, wr, tokens,
                       routing=wl.routing)
