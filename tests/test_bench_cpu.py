"""Host logic of bench.py, without a GPU: the one-GPU guard, the algorithmic
byte model behind the roofline figures, and the rule that a stored HBM
traffic figure is used only while the kernel sources it was taken on are
unchanged."""

import json
import os
import subprocess
import sys

import pytest

import bench
import bit_quantized_moe_gemv_amd as bq
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


@pytest.mark.parametrize("fmt,books", [(W.FMT_MXFP4, 0), (W.FMT_VQ13R8, (8192 + 256) * 8 * 2),
                                       (W.FMT_VQ13, 8192 * 8 * 2)])
def test_expert_bytes_match_the_packed_layout(fmt, books):
    """Per-expert gate/up + down bytes of the model times the expert count,
    plus the codebooks, is the packed size the C ABI reports."""
    wl = W.DECODE.replace(fmt=fmt)
    one = bench.algorithmic(wl, 1, 1)
    H, I, k = wl.hidden, wl.inter, wl.top_k
    gu = one["gateup_bytes"] - H * 2 - k * I * 4
    dn = one["down_bytes"] - k * I * 4 - H * 4
    assert wl.experts * (gu + dn) + books == bq.packed_size(H, I, wl.experts, k, fmt=fmt)


def test_decode_roofline_unit():
    """The dominant decode kernel's algorithmic bytes per launch: 8 experts'
    gate/up weights, the token's x and its 8 h rows."""
    a = bench.algorithmic(W.DECODE, 8, 1)
    assert a["gateup_bytes"] == 8 * 2 * 2048 * 4096 * 17 // 32 + 4096 * 2 + 8 * 2048 * 4 \
        == 71376896
    p = bench.algorithmic(W.PREFILL, 256, 2048)
    assert p["gateup_flops"] == 2 * 2048 * 8 * 2 * 2048 * 4096


def test_unknown_format_is_an_error():
    with pytest.raises(ValueError):
        bench.algorithmic(W.DECODE.replace(fmt=9), 8, 1)


def test_traffic_figure_follows_the_sources(tmp_path, monkeypatch):
    rec = {"kernel": "k", "source_sha256": bench._src_hash("decode.hip", "moe_internal.h"),
           "hbm_bytes_per_launch": 12345}
    (tmp_path / "k_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench._traffic("k", ("decode.hip", "moe_internal.h"), 1) == 12345
    assert bench._traffic("k", ("decode.hip",), 1) is None  # a different source set
    rec["source_sha256"] = "0" * 64
    (tmp_path / "k_traffic.json").write_text(json.dumps(rec))
    assert bench._traffic("k", ("decode.hip", "moe_internal.h"), 1) is None
    assert bench._traffic("missing", ("decode.hip",), 1) is None
