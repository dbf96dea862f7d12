"""The layer shape is pinned by totals the model cards print
(tests/golden/page_payloads.txt): hidden 4096, expert intermediate 2048,
top-8 routing over 256 experts, 47 MoE layers."""

import os

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_payloads.txt")


def _golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v) if "." in v else int(v)
    return vals


def test_payload_totals_fix_hidden_and_intermediate():
    g = _golden()
    moe_layers = g["layers"] - g["dense_layers"]
    assert moe_layers == 47
    h, i, e = W.DECODE.hidden, W.DECODE.inter, W.DECODE.experts
    assert e == g["routed_experts"] and W.DECODE.top_k == g["active_experts"]
    # IQ2_XXS gate/up at 2.0625 bit/weight, IQ2_XS down at 2.3125 bit/weight
    assert moe_layers * e * 2 * i * h * 2.0625 / 8 == g["routed_gate_up_payload_bytes"]
    assert moe_layers * e * h * i * 2.3125 / 8 == g["routed_down_payload_bytes"]
    assert round(moe_layers * e * 3 * i * h / 1e9, 2) == g["routed_params_billions"]
    assert moe_layers * e * 3 == g["routed_expert_matrices"]
    assert moe_layers * e == g["layer_expert_slots"]
    assert moe_layers * 3 == g["expert_projections"]
    assert g["staged_experts"] * i * 2 == g["staged_intermediate_bytes"]


def test_mxfp4_layer_size():
    # 4.25 bit per weight (4-bit element + 8-bit scale per 32)
    wl = W.DECODE
    assert wl.packed_bytes == 3422552064
    assert wl.packed_bytes * 8 / (wl.experts * 3 * wl.inter * wl.hidden) == 4.25
