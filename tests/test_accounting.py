"""Accounting closed forms against the numbers the pages print
(tests/golden/page_figures.json, each entry cited there)."""

import json
import os

from cross_entropy_lm_amd import accounting as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "page_figures.json")))


def test_traffic_model_saving():
    g = GOLD["traffic_model"]
    t = A.dw_table_traffic(g["V"], g["D"], g["chunks"])
    assert t["saving"] / A.GiB == g["saving_GiB"]
    assert t["current"] - t["candidate"] == t["saving"]
    assert t["candidate"] == 4 * g["V"] * g["D"] * (1 + 2 * g["chunks"])


def test_chunk_sweep_rows():
    g = GOLD["chunk_sweep_rows"]
    for elems, rows in g["elems_to_rows"].items():
        assert A.rows_per_chunk(int(elems), g["V"]) == rows


def test_gradient_and_transient_bytes():
    g = GOLD["gradient_bytes"]
    for rows, gib in g["rows_to_GiB_2dp"].items():
        assert round(A.logits_bytes(int(rows), g["V"], 2) / A.GiB, 2) == gib
    o = GOLD["old_vjp_transient"]
    assert round(o["N"] * o["V"] * o["bytes_per_logit"] / A.GiB, 2) == o["GiB_2dp"]


def test_dw_temporaries():
    g = GOLD["dw_temporaries"]
    assert A.dw_temporary_bytes(g["V"], g["H"], 2) / A.MiB == g["MiB_16bit"]
    assert A.dw_temporary_bytes(g["V"], g["H"], 4) / A.MiB == g["MiB_fp32"]


def test_throughput_definition():
    g = GOLD["throughput"]
    # the printed median is rounded to 0.01 ms, which moves tokens/s by up to ~0.2
    lo = A.tokens_per_s(g["N"], g["median_ms"] + 0.005)
    hi = A.tokens_per_s(g["N"], g["median_ms"] - 0.005)
    # and the printed tokens/s is itself rounded to 0.1: the two intervals must overlap
    assert lo <= g["tokens_per_s_1dp"] + 0.05 and g["tokens_per_s_1dp"] - 0.05 <= hi


def test_flop_counts():
    assert A.linear_fwd_bwd_flops(16384, 4096, 32000) == 4 * A.contraction_flops(16384, 32000, 4096)
    assert A.linear_model_flops(1, 1, 1) == 6
    assert A.logits_only_bytes(32768, 151936, 2) == 3 * 32768 * 151936 * 2
