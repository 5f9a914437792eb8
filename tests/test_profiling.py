"""The HBM-traffic summary lookup on the CPU: a figure is reported only for
the device sources it was taken with and for the exact kernel instance the
plan launches."""
import json
import os

import pytest

import row_reductions_amd as lr
from row_reductions_amd import profiling

# the demangled parameter list of every kernel entry
ENTRY = "(float const*, long, int, int, int, int, float const*, float const*, float const*, lr::KArgs)"
SUMMARY = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles",
                       "hbm_traffic_768x6144.json")


def test_kernel_names_follow_the_plan():
    F = lr.lr_device_facts_mi355x()
    p = lr.lr_plan_for_device(F, "rmsnorm", 768, 6144, "unordered_tree", 1)
    p.family, p.chunks_per_lane = lr.LR_FAMILY_CACHE, 3
    assert profiling.kernel_name(1, p, True, 1) == "void lr::k_cache<1, 3, true, 1>" + ENTRY
    p.family = lr.LR_FAMILY_STREAM
    assert profiling.kernel_name(0, p, False, 0) == "void lr::k_stream<0, false>" + ENTRY
    p.family = lr.LR_FAMILY_SPLIT
    assert profiling.kernel_name(0, p, True, 0) is None


def test_lookup_requires_matching_sources_and_instance(tmp_path):
    rec = {"op": "softmax", "traffic_bytes": 1.0}
    good = tmp_path / "good.json"
    good.write_text(json.dumps({"csrc_sha256": profiling.csrc_hash(),
                                "kernels": {"void lr::k_cache<0, 6, true, 0>" + ENTRY: rec}}))
    assert profiling.lookup(str(good), "softmax")["traffic_bytes"] == 1.0
    assert profiling.lookup(str(good), "softmax", "void lr::k_cache<0, 6, true, 0>" + ENTRY) is not None
    assert profiling.lookup(str(good), "softmax", "void lr::k_cache<0, 4, true, 0>" + ENTRY) is None
    assert profiling.lookup(str(good), "rmsnorm") is None
    stale = tmp_path / "stale.json"
    stale.write_text(json.dumps({"csrc_sha256": "0" * 64, "kernels": {"k": rec}}))
    assert profiling.lookup(str(stale), "softmax") is None
    assert profiling.lookup(str(tmp_path / "missing.json"), "softmax") is None


def test_committed_summary_covers_the_planned_kernels():
    with open(SUMMARY) as f:
        s = json.load(f)
    if s["csrc_sha256"] != profiling.csrc_hash():
        pytest.skip("kernels changed since the counters were taken (the bench reports traffic: null)")
    F = lr.lr_device_facts_mi355x()
    for op, pm in (("softmax", 0), ("rmsnorm", 1), ("layernorm", 1)):
        p = lr.lr_plan_for_device(F, op, 768, 6144, "unordered_tree", 1)
        r = profiling.lookup(SUMMARY, op, profiling.kernel_name(lr.OPS[op], p, True, pm))
        assert r is not None, op
        # no re-reads: within 2% of the algorithmic 37,748,736 B
        assert abs(r["traffic_bytes"] / 37748736 - 1) < 0.02, (op, r["traffic_bytes"])


TRACE = os.path.join(os.path.dirname(SUMMARY), "kernel_trace_768x6144.json")


def test_committed_trace_covers_the_planned_kernels():
    """The kernel-trace summary the bench's frac_trace reads names the very
    instances the plans launch, with averages no shorter than a transfer of
    the algorithmic bytes at 8 TB/s could take."""
    with open(TRACE) as f:
        s = json.load(f)
    if s["csrc_sha256"] != profiling.csrc_hash():
        pytest.skip("kernels changed since the trace was taken (the bench reports frac_trace: null)")
    F = lr.lr_device_facts_mi355x()
    for op, pm in (("softmax", 0), ("rmsnorm", 1), ("layernorm", 1)):
        p = lr.lr_plan_for_device(F, op, 768, 6144, "unordered_tree", 1)
        r = profiling.lookup(TRACE, op, profiling.kernel_name(lr.OPS[op], p, True, pm))
        assert r is not None, op
        assert r["avg_us"] > 37748736 / 8e12 * 1e6 and r["dispatches"] > 1000, (op, r)
