"""Workload parameters against what the POP notes print."""
import json
import os

from online_structured_ffn_amd.configs import LLAMA2_7B, LLAMA2_7B_B16, WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_llama_ffn_rate_from_global_budget():
    g = json.load(open(os.path.join(GOLDEN, "ffn_budget.json")))
    d, dff = g["d"], g["d_ff"]
    attn, ffn = 4 * d * d, 3 * d * dff
    r_ffn = g["global_rate"] * (attn + ffn) / ffn
    assert round(100 * r_ffn, 1) == g["printed_ffn_rate_percent"]
    assert abs(r_ffn - g["workload_r_ffn"]) < 5e-4
    assert LLAMA2_7B.r == LLAMA2_7B_B16.r == g["workload_r_ffn"]


def test_ablation_table_ratios_consistent():
    # POP notes, ablation table: extra FFN TFLOPs over dense, and the printed percentages
    rows = [(22.09, 0.63, 2.85), (22.09, 7.32, 33.1), (28.75, 9.56, 33.3), (28.75, 1.00, 3.48)]
    for dense, extra, pct in rows:
        assert abs(100 * extra / dense - pct) < 0.05


def test_workload_shapes_are_vector_friendly():
    for w in WORKLOADS:
        assert w.d % 8 == 0 and w.d_ff > 0 and 0 <= w.r < 1 and w.gamma == 0.1
