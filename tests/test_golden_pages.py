"""The code's constants and byte accounting against values printed on the pages
(tests/golden/pages_constants.json, each entry citing its page and section)."""
import json
import os

from layernorm_reduction_amd import workloads as W

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def test_layernorm_eps():
    assert W.LN_EPS == GOLDEN["layernorm_eps"]["value"]


def test_softmax_sweep_is_the_template_list():
    assert list(W.SOFTMAX_TK_SWEEP) == GOLDEN["softmax_bw_row_length_templates"]["value"]


def test_attention_probability_traffic_reproduces_805_mb():
    g = GOLDEN["attention_probability_traffic"]
    total = W.attention_probability_traffic(g["B"], g["H"], g["T"], g["bytes_per_element"], g["layers"])
    assert total == 805_306_368
    assert round(total / 1e6) == g["megabytes"]
    # The same bytes are the probability write of the forward plus the read of the backward
    # in this library's per-op accounting (fp32 storage, one layer, times 6 layers).
    s = g["bytes_per_element"]
    E = g["B"] * g["H"] * g["T"] * g["T"]
    per_layer = E * s + E * s   # y written by softmax_fw, y read by softmax_bw
    assert per_layer * g["layers"] == total
    assert W.softmax_fw_bytes(g["B"], g["H"], g["T"], g["T"], s, has_mask=False) == 2 * E * s
    assert W.softmax_bw_bytes(g["B"], g["H"], g["T"], g["T"], s) == 3 * E * s


def test_gpt2_shapes_of_workload_two():
    g = GOLDEN["gpt2_training_shape"]
    assert g["B"] * g["T"] == g["tokens_per_step"]
    [s], [ln] = W.workload2()
    assert (s.B, s.H, s.Tq, s.Tk) == (g["B"], g["H"], g["T"], g["T"])
    assert (ln.N, ln.C) == (g["B"] * g["T"], g["C"])


def test_fused_add_three_counts():
    g = GOLDEN["fused_add_three_example"]
    # C = A + B then E = C + D: each kernel loads two operands and stores one result.
    assert (2 + 2, 1 + 1) == (g["unfused_loads"], g["unfused_stores"])
    assert (3, 1) == (g["fused_loads"], g["fused_stores"])
