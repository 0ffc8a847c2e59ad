"""The CPU legs of bench.py (the oracle timed as a reported baseline), on a
short budget: the single-threaded sample and the process-pool sample report
the JSON fields the bench line carries, with the cores they used."""
import os
import sys

import workloads as wl

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_cpu_baselines_report_their_cores():
    bt = wl.make("quest_gqa_32k")
    one = bench.cpu_baseline(bt, 0.2)
    assert one["cores"] == 1 and one["kind"] == "oracle" and one["value"] > 0
    par = bench.cpu_baseline_parallel(bt, 0.2, 4)
    assert par["cores"] == 4 and par["kind"] == "oracle" and par["value"] > 0
    assert "4 single-threaded processes" in par["sample"]


def test_parallel_baseline_needs_two_units():
    bt = wl.make("tiny_f32")   # one (sequence, KV head) unit
    assert bench.cpu_baseline_parallel(bt, 0.1, 8) is None
