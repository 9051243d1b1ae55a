"""The benchmark's flop and byte accounting, pinned to the FlagOS-OP page's
perf-gate row (a printed time and rate for one causal call)."""

import json
import os

import bench
import sdpa_workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_perf_gate.json")


def test_flops_reproduce_page_perf_gate():
    g = json.load(open(GOLDEN))
    r = g["reading"]
    f = bench.algorithmic_flops(1, r["BH"], r["Sq"], r["Skv"], r["D"], r["D"], r["causal"])
    # the printed time has 3 significant digits: the rate must fall inside its rounding interval
    lo = f / ((g["ms"] + 0.0005) * 1e-3) / 1e12
    hi = f / ((g["ms"] - 0.0005) * 1e-3) / 1e12
    assert lo <= g["tflops"] <= hi


def test_bytes_of_the_timed_workload():
    w = W.BY_NAME["prefill_2k_d128_bf16_causal"]
    b = bench.algorithmic_bytes(w)
    assert b["p"] == 2 * 16 * 2048 * 2048 * 2
    assert b["total"] == b["p"] + 4 * (2 * 16 * 2048 * 128 * 2) + 2 * 16 * 2048 * 4
    assert abs(bench.algorithmic_flops(2, 16, 2048, 2048, 128, 128, True) - 34.36e9) < 0.01e9
