"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: the
plain C reference (oracle/oracle.c) is compiled with both sanitizers into a
small driver (oracle_sanitize_driver.c) that runs the routing, the grouping,
the matrix decoders and the whole layer for tiny MXFP4, VQ13R8 and VQ13
layers.  Any sanitizer report fails the test."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

SANITIZERS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer"]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-g", "-O1", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           *SANITIZERS, "-Wall", "-o", exe,
           os.path.join(HERE, "oracle_sanitize_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
           "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="abort_on_error=0:halt_on_error=1:detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    report = res.stdout + res.stderr
    assert res.returncode == 0, report
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
    for name in ("mxfp4", "vq13r8", "vq13"):
        assert f"{name} ok" in res.stdout
    assert "0 failures" in res.stdout
