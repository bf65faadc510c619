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


def test_bench_per_launch_kind_flops():
    """The bench's per-kind flop of the single call adds up to three N x V x D
    contractions for every chunking and schedule, and splits as the schedule
    says: with overlap only chunk 0's forward has a launch of its own; with
    groups of G chunks the last launch holds the dW of the last group."""
    import sys
    sys.path.insert(0, ROOT)
    import bench

    D, V = 64, 1000
    for N, C in ((16384, 2048), (300, 128), (300, 7), (4096, 512), (5, 5), (1000, 300), (8192, 110)):
        K = -(-N // C)
        ck = [min(C, N - k * C) for k in range(K)]
        for overlap, G, gdh in ((False, 1, False), (False, 2, False), (True, 1, False), (True, 2, False),
                                (True, 2, True), (False, 2, True), (True, 4, True), (True, 7, False),
                                (False, 7, False), (True, 3, True)):
            f = bench.fused_step_flops(N, D, V, C, K, overlap, G, gdh)
            assert sum(f.values()) == 6 * N * V * D, (N, C, overlap, G, gdh)
            if not gdh:
                if overlap:
                    assert f["fwd_lse"] == 2 * min(C, N) * V * D
                    if G > 1 and K >= 2:
                        grp = sum(ck[K - 1 - (K - 1) % G:])  # the last group's tokens
                        assert f["dh_dw"] == 2 * ck[-1] * V * D + 2 * grp * V * D
                else:
                    assert f["fwd_lse"] == 2 * N * V * D and f.get("dh_dw_fwd", 0) == 0
            elif overlap and K >= 3 and G > 1:
                # group dH: chunk 0's forward, and the launches of chunks that do
                # not end a group carry only the next chunk's forward
                fwd_only = sum(ck[k + 1] for k in range(K - 1) if k % G != G - 1)
                assert f["fwd_lse"] == 2 * V * D * (ck[0] + fwd_only)
