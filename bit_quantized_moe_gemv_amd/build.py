"""Build libbqmoe.so (all HIP sources, gfx950) in-tree with hipcc."""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbqmoe.so")
SOURCES = ["abi.hip", "route.hip", "decode.hip", "prefill.hip", "vq_prefill.hip", "vq_decode.hip",
           "measure.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # the router's summation order is part of the contract: no contraction
    "-ffp-contract=off",
    # no packed-fp32 instructions anywhere in this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l]
    return res.returncode, msgs


def build(verbose: bool = False) -> str:
    """Compile every source to an object file (in parallel), then link the
    shared library; the objects go to a build folder beside the sources."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    jobs = []
    for s in SOURCES:
        obj = os.path.join(objdir, s.replace(".hip", ".o"))
        jobs.append((obj, [HIPCC, *compile_flags, *inc, "-c", "-o", obj, os.path.join(CSRC, s)]))
    if verbose:
        for _, cmd in jobs:
            print(" ".join(cmd), flush=True)
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(workers) as pool:
        results = list(pool.map(lambda j: _run(j[1]), jobs))
    failed = False
    for (obj, _), (rc, msgs) in zip(jobs, results):
        if rc != 0 or (verbose and msgs):
            sys.stderr.write("\n".join(msgs) + "\n")
        failed |= rc != 0
    if failed:
        raise RuntimeError("hipcc failed building libbqmoe.so")
    tmp = LIB + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in jobs]]
    if verbose:
        print(" ".join(link), flush=True)
    rc, msgs = _run(link)
    if rc != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed linking libbqmoe.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
