"""CPU check of the ranking helpers of the GPU top-k selections: a NaN logit
(from non-finite activations) ranks as -inf, and the unsigned key the batch-1
set selection compares is monotone in the float value with -0 == +0.  The
helpers are __host__ __device__, so route_keys_host.hip runs them as a plain
host program; no GPU call is made."""

import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_selection_value_and_order_key(tmp_path):
    exe = str(tmp_path / "route_keys_host")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "bit_quantized_moe_gemv_amd", "csrc"),
           "-o", exe, os.path.join(HERE, "route_keys_host.hip")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout
