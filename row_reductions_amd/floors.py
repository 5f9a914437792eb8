"""Floors of the two launch-bound workloads, measured by scaling one
dimension and fitting a line.

    python -m row_reductions_amd.floors [--json]

ordered_fold RMSNorm, 256 rows: one wavefront folds each row as a single
dependent FP32 add chain (the pages' fold_left, "TIRx Metal reduction
lowering", section 1), so the time grows with cols at the chain's rate.  The
fit t = a + b * cols over cols = 768 .. 12288 gives the chain's cost per
element b (and, at 2.4 GHz, the cycles per dependent add) and the fixed part
a; 256 x 3072 is then a + 3072 b.

LayerNorm, 64 rows of 12289 floats: one workgroup per row, so only 64 of the
256 compute units work.  The fit over cols = 1537 .. 24577 (misaligned rows,
as at 12289) gives the fixed part and the rate one workgroup streams its row
at; the same row count at 4x the rows (256 rows, every CU busy) shows what
the width costs.  A one-row, 64-column call is the smallest launch: the
fixed cost of any kernel here.

Every point is timed as HIP-graph replays (200 launches per graph, resident
inputs), median of five batches of >= 30 ms after >= 200 ms of warm-up, as
the bench times its launch-bound workloads.

The copy floor at 768 x 6144, cold: under the plan each of softmax, RMSNorm
and LayerNorm launches with, the row copy (lr_copy_rows_f32: the same
workgroups, reads and stores, no arithmetic between them), each wave storing
as soon as its reads land, and with the reads of the whole workgroup landed
and one barrier before the first store (the reductions' shape), beside the
operation itself.  The copy's time is what moving the bytes through that
launch shape costs; the difference is the operation's own work.  Then the
copy, both ways, under every one-row CACHE plan it compiles: its fastest is
the floor of a launch of this size.

RMSNorm and LayerNorm, 768 x 6144, with and without their per-column
parameters (gamma; gamma and beta), each at the plan the library picks for
that call (RMSNorm without gamma has a plan of its own) and at six waves per
row, cold (32 rotating buffer sets, as the bench): the
difference is what reading the parameters after the row's reductions costs
a launch, although they add no HBM traffic (they are L2 hits).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import sys
import time

import numpy as np
import torch

import row_reductions_amd as lr

N_GRAPH = 200


def _time_graph(fn, samples=5, sample_ms=30.0, warmup_ms=200.0):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        lr.check(fn(side.cuda_stream), "warm-up call")
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            for _ in range(N_GRAPH):
                fn(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < warmup_ms:
        graph.replay()
        torch.cuda.synchronize()
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    graph.replay()
    z.record()
    torch.cuda.synchronize()
    reps = max(1, int(sample_ms / a.elapsed_time(z)) + 1)
    vals = []
    for _ in range(samples):
        graph.replay()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            graph.replay()
        z.record()
        torch.cuda.synchronize()
        vals.append(a.elapsed_time(z) * 1e3 / (reps * N_GRAPH))
    vals.sort()
    del graph
    return vals[len(vals) // 2]


def _time_cold(fn, sets, samples=7, sample_ms=30.0, warmup_ms=200.0):
    """Median us per launch of fn(i) over batches of back-to-back launches
    (i picks one of `sets` buffer sets), the bench's per-op protocol."""
    i = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < warmup_ms:
        for _ in range(64):
            lr.check(fn(i % sets), "launch")
            i += 1
        torch.cuda.synchronize()
    n = int(sample_ms / 7e-3) + 1
    vals = []
    for _ in range(samples):
        for _ in range(8):
            fn(i % sets)
            i += 1
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn(i % sets)
            i += 1
        z.record()
        torch.cuda.synchronize()
        vals.append(a.elapsed_time(z) * 1e3 / n)
    vals.sort()
    return vals[len(vals) // 2]


def _fit(xs, ts):
    b, a = np.polyfit(np.asarray(xs, float), np.asarray(ts, float), 1)
    return float(a), float(b)


def counter_launches(n: int) -> int:
    """Softmax, and RMSNorm and LayerNorm with and without their parameters,
    768 x 6144 at the library's plans, n cold launches each (32 rotating
    buffer sets) and no timing: the program to run under a counter pass,
    whose per-kernel figures then belong to one launch configuration each."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev).manual_seed(0)
    rows, cols, sets = 768, 6144, 32
    xs = [torch.randn(rows, cols, device=dev, generator=g) for _ in range(sets)]
    ys = [torch.empty_like(t) for t in xs]
    gm = torch.rand(cols, device=dev, generator=g) + 0.5
    bt = torch.randn(cols, device=dev, generator=g) * 0.1
    sh = torch.cuda.current_stream().cuda_stream
    xp, yp = [t.data_ptr() for t in xs], [t.data_ptr() for t in ys]
    gp, bp = gm.data_ptr(), bt.data_ptr()
    calls = [
        ("softmax", lambda k: lr.lib.lr_softmax_f32(xp[k], yp[k], rows, cols, 0, sh)),
        ("rmsnorm with gamma", lambda k: lr.lib.lr_rmsnorm_f32(xp[k], gp, yp[k], rows, cols, 1e-6, 0, sh)),
        ("rmsnorm without", lambda k: lr.lib.lr_rmsnorm_f32(xp[k], None, yp[k], rows, cols, 1e-6, 0, sh)),
        ("layernorm with gamma, beta", lambda k: lr.lib.lr_layernorm_f32(xp[k], gp, bp, yp[k], rows, cols, 1e-5, 0, sh)),
        ("layernorm without", lambda k: lr.lib.lr_layernorm_f32(xp[k], None, None, yp[k], rows, cols, 1e-5, 0, sh)),
    ]
    for name, fn in calls:
        for i in range(n):
            lr.check(fn(i % sets), name)
        torch.cuda.synchronize()
        print(f"{name}: {n} launches", flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--json", action="store_true")
    ap.add_argument("--counter-launches", type=int, default=0, metavar="N",
                    help="only launch the 768x6144 norms with and without parameters (and softmax) N times "
                         "each, untimed: the program for a counter pass")
    args = ap.parse_args(argv)
    if args.counter_launches:
        return counter_launches(args.counter_launches)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev).manual_seed(0)
    out = {}

    # the smallest launch
    x1 = torch.randn(1, 64, device=dev, generator=g)
    y1 = torch.empty_like(x1)
    out["tiny_softmax_1x64_us"] = _time_graph(lambda sh: lr.lr_softmax_f32(x1, y1, 1, 64, 0, sh))

    # ordered_fold RMSNorm, 256 rows
    fold = {}
    for cols in (768, 1536, 3072, 6144, 12288):
        x = torch.randn(256, cols, device=dev, generator=g)
        gm = torch.rand(cols, device=dev, generator=g) + 0.5
        y = torch.empty_like(x)
        fold[cols] = _time_graph(lambda sh, x=x, gm=gm, y=y, c=cols: lr.lr_rmsnorm_f32(x, gm, y, 256, c, 1e-6, 1, sh))
        print(f"ordered_fold rmsnorm 256x{cols}: {fold[cols]:.3f} us", flush=True)
    a, b = _fit(list(fold), list(fold.values()))
    out["ordered_fold_rmsnorm_256"] = {
        "us": {str(k): round(v, 3) for k, v in fold.items()},
        "fit_fixed_us": round(a, 3), "fit_us_per_element": b, "fit_cycles_per_element_at_2.4GHz": round(b * 2400, 2),
        "fit_at_3072_us": round(a + 3072 * b, 3)}
    x = torch.randn(256, 3072, device=dev, generator=g)
    gm = torch.rand(3072, device=dev, generator=g) + 0.5
    y = torch.empty_like(x)
    out["unordered_rmsnorm_256x3072_us"] = round(
        _time_graph(lambda sh: lr.lr_rmsnorm_f32(x, gm, y, 256, 3072, 1e-6, 0, sh)), 3)

    # LayerNorm, 64 misaligned rows, and 256 rows of the same width
    ln = {}
    for cols in (1537, 3073, 6145, 12289, 24577):
        x = torch.randn(64, cols, device=dev, generator=g) * 2 + 3
        gm = torch.rand(cols, device=dev, generator=g) + 0.5
        bt = torch.randn(cols, device=dev, generator=g) * 0.1
        y = torch.empty_like(x)
        ln[cols] = _time_graph(lambda sh, x=x, gm=gm, bt=bt, y=y, c=cols:
                               lr.lr_layernorm_f32(x, gm, bt, y, 64, c, 1e-5, 0, sh))
        print(f"layernorm 64x{cols}: {ln[cols]:.3f} us", flush=True)
    a, b = _fit(list(ln), list(ln.values()))
    row_bytes_per_us = 8.0 / (b * 1e-6) / 1e6  # bytes of one row (read + write) per element / us per element
    out["layernorm_64_rows"] = {
        "us": {str(k): round(v, 3) for k, v in ln.items()},
        "fit_fixed_us": round(a, 3), "fit_us_per_element": b,
        "fit_at_12289_us": round(a + 12289 * b, 3),
        "per_workgroup_rate_GBps": round(row_bytes_per_us / 1e3, 1)}
    x = torch.randn(256, 12289, device=dev, generator=g) * 2 + 3
    gm = torch.rand(12289, device=dev, generator=g) + 0.5
    bt = torch.randn(12289, device=dev, generator=g) * 0.1
    y = torch.empty_like(x)
    out["layernorm_256x12289_us"] = round(
        _time_graph(lambda sh: lr.lr_layernorm_f32(x, gm, bt, y, 256, 12289, 1e-5, 0, sh)), 3)
    xr = x[:64].contiguous()
    sums = torch.empty(64, device=dev)
    out["row_sum_64x12289_us"] = round(_time_graph(lambda sh: lr.lr_row_sum_f32(xr, sums, 64, 12289, 0, sh)), 3)
    # gamma / beta at 768 x 6144, cold
    rows, cols, sets = 768, 6144, 32
    xs = [torch.randn(rows, cols, device=dev, generator=g) for _ in range(sets)]
    ys = [torch.empty_like(t) for t in xs]
    gm = torch.rand(cols, device=dev, generator=g) + 0.5
    bt = torch.randn(cols, device=dev, generator=g) * 0.1
    facts = lr.lr_device_facts_query()
    sh = torch.cuda.current_stream().cuda_stream
    xp, yp = [t.data_ptr() for t in xs], [t.data_ptr() for t in ys]
    gp, bp = gm.data_ptr(), bt.data_ptr()
    par = {}
    for op in ("rmsnorm", "layernorm"):
        six = next(p for p in lr.lr_plan_enumerate(facts, op, rows, cols, "unordered_tree", 1)
                   if p.family == lr.LR_FAMILY_CACHE and p.waves_per_row == 6 and p.rows_per_block == 1
                   and p.lanes_per_row == 384)
        for pname, plan in (("auto", lr.lr_plan_query(op, rows, cols, "unordered_tree")), ("S6", six)):
            pp = ctypes.byref(plan)
            for with_p in (True, False):
                # raw calls on precomputed pointers: the host must outpace the
                # GPU's 7 us per launch
                g_, b_ = (gp, bp) if with_p else (None, None)
                if pname == "auto":
                    # the typed call: a norm without its parameters may take
                    # a plan of its own
                    if op == "rmsnorm":
                        fn = (lambda k, g_=g_: lr.lib.lr_rmsnorm_f32(xp[k], g_, yp[k], rows, cols, 1e-6, 0, sh))
                    else:
                        fn = (lambda k, g_=g_, b_=b_: lr.lib.lr_layernorm_f32(
                            xp[k], g_, b_, yp[k], rows, cols, 1e-5, 0, sh))
                elif op == "rmsnorm":
                    fn = (lambda k, pp=pp, g_=g_: lr.lib.lr_rmsnorm_f32_with_plan(
                        xp[k], g_, yp[k], rows, cols, 1e-6, 0, pp, sh))
                else:
                    fn = (lambda k, pp=pp, g_=g_, b_=b_: lr.lib.lr_layernorm_f32_with_plan(
                        xp[k], g_, b_, yp[k], rows, cols, 1e-5, 0, pp, sh))
                key = f"{op}_{pname}_{'params' if with_p else 'no_params'}"
                par[key] = round(_time_cold(fn, sets), 3)
                print(f"{key}: {par[key]} us", flush=True)
    out["params_768x6144_cold_us"] = par
    # the copy floor: each operation's own plan with the row copy (the same
    # reads and stores, nothing between them) in place of the operation
    cp = {}
    for op in ("softmax", "rmsnorm", "layernorm"):
        plan = lr.lr_plan_query(op, rows, cols, "unordered_tree")
        pp = ctypes.byref(plan)
        if op == "softmax":
            fn = lambda k, pp=pp: lr.lib.lr_softmax_f32_with_plan(xp[k], yp[k], rows, cols, 0, pp, sh)
        elif op == "rmsnorm":
            fn = lambda k, pp=pp: lr.lib.lr_rmsnorm_f32_with_plan(xp[k], gp, yp[k], rows, cols, 1e-6, 0, pp, sh)
        else:
            fn = lambda k, pp=pp: lr.lib.lr_layernorm_f32_with_plan(xp[k], gp, bp, yp[k], rows, cols, 1e-5, 0, pp, sh)
        copy = lambda k, pp=pp: lr.lib.lr_copy_rows_f32(xp[k], yp[k], rows, cols, pp, 0, sh)
        copy_sync = lambda k, pp=pp: lr.lib.lr_copy_rows_f32(xp[k], yp[k], rows, cols, pp, 1, sh)
        rec = {"plan": f"S={plan.waves_per_row}, {plan.chunks_per_lane} chunks"}
        for _ in range(2):  # each config twice, interleaved: the lower median of the two
            for key, f in (("op_us", fn), ("copy_us", copy), ("copy_sync_us", copy_sync)):
                t = _time_cold(f, sets)
                rec[key] = round(min(rec.get(key, t), t), 3)
        rec["gap_to_copy_sync_us"] = round(rec["op_us"] - rec["copy_sync_us"], 3)
        for key in ("op_us", "copy_us", "copy_sync_us"):
            rec[key.replace("_us", "_frac_of_8TBps")] = round(2 * rows * cols * 4 / (rec[key] * 1e-6) / 8e12, 4)
        cp[op] = rec
        print(f"copy floor {op}: {rec}", flush=True)
    out["copy_768x6144_cold_us"] = cp
    # the same copy under every one-row CACHE plan the copy compiles: the
    # fastest a launch of this shape moves these bytes
    sweep = {}
    for p in lr.lr_plan_enumerate(facts, "softmax", rows, cols, "unordered_tree", 1):
        if (p.family != lr.LR_FAMILY_CACHE or p.rows_per_block != 1 or p.lanes_per_row != 64 * p.waves_per_row
                or p.chunks_per_lane not in (1, 2, 3, 4, 6, 8)):
            continue
        pp = ctypes.byref(p)
        key = f"S={p.waves_per_row}, {p.chunks_per_lane} chunks"
        sweep[key] = {f"sync{sy}": round(_time_cold(lambda k, pp=pp, sy=sy: lr.lib.lr_copy_rows_f32(
            xp[k], yp[k], rows, cols, pp, sy, sh), sets), 3) for sy in (0, 1)}
        print(f"copy sweep {key}: {sweep[key]}", flush=True)
    best = min(((v, k, m) for k, r in sweep.items() for m, v in r.items()))
    out["copy_sweep_768x6144_cold_us"] = {"plans": sweep, "best_us": best[0], "best_plan": best[1],
                                          "best_mode": best[2],
                                          "best_frac_of_8TBps": round(2 * rows * cols * 4 / (best[0] * 1e-6) / 8e12, 4)}
    del xs, ys
    out["tiny_softmax_1x64_us"] = round(out["tiny_softmax_1x64_us"], 3)
    print(json.dumps(out) if args.json else json.dumps(out, indent=1), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
