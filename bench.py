"""Benchmark of the FP32 row-reduction hot path on one MI355X.

One step = softmax, RMSNorm and LayerNorm, each on a 768 x 6144 FP32 tensor
(x ~ N(0,1), gamma ~ U(0.5,1.5), beta ~ N(0, 0.1^2), eps 1e-6 / 1e-5), launched
through the C ABI on the current torch stream.  Inputs are device-resident
before timing.  By default every launch reads a different buffer set out of
32 rotating sets (1.2 GB in total, larger than the 256 MB Infinity Cache and
the L2s), so each launch streams its tensor from HBM ("cold").

Printed: one JSON line with throughput (GB/s of algorithmic bytes = tensor
read + tensor write per op), per-op microseconds, the roofline record of the
dominant kernel, the oracle's CPU baseline and, as context, warm-cache and
cross-entropy 4096 x 32000 figures.

Per-op times follow the measurement protocol of the pages' whole-launch cost
notes, whatever --steps is: at least 200 ms of warm-up launches, then nine
samples, each a batch of back-to-back launches of that op alone lasting at
least 30 ms between two HIP events on the launch stream; the median is
reported with the [min, max] range.  The roofline's average launch duration
is that median.

    python bench.py [--steps K] [--warmup W] [--warm] [--no-cpu-baseline]
                    [--no-extra] [--copy-probe]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

ROWS, COLS = 768, 6144
OPS = ("softmax", "rmsnorm", "layernorm")
EPS = {"rmsnorm": 1e-6, "layernorm": 1e-5}
HBM_PEAK_GBS = 8000.0
METRIC = "µs/op + achieved HBM GB/s (% of peak), FP32 softmax/RMSNorm/LayerNorm 768×6144"
# The pages' M1 Max command-buffer medians at 768x6144 (softmax, RMSNorm,
# LayerNorm): 57.414 + 60.753 + 75.251 us for the three ops' algorithmic bytes.
PAGES_M1MAX_STEP_US = 57.414 + 60.753 + 75.251


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_768x6144.json")
TRACE_SUMMARY = os.path.join(ROOT, "profiles", "kernel_trace_768x6144.json")


def traffic_bytes(lr, op: str):
    """HBM bytes per launch of `op` from the committed FETCH_SIZE / WRITE_SIZE
    summary (copy-calibrated), or None when the kernels changed since or the
    summary was taken for another kernel instance than this plan's."""
    from row_reductions_amd import profiling
    plan = lr.lr_plan_query(op, ROWS, COLS, "unordered_tree")
    params = {"softmax": 0, "rmsnorm": 1, "layernorm": 1}[op]  # gamma (and beta) present
    kernel = profiling.kernel_name(lr.OPS[op], plan, True, params)
    rec = profiling.lookup(TRAFFIC_SUMMARY, op, kernel)
    return None if rec is None else round(rec["traffic_bytes"])


WARMUP_MS = 200.0
SAMPLE_MS = 30.0
SAMPLES = 9


def progress(msg: str) -> None:
    """A progress line on stderr (the JSON result alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_batches(torch, stream, launch, samples: int = SAMPLES, sample_ms: float = SAMPLE_MS,
                 warmup_ms: float = WARMUP_MS, calib: int = 200) -> dict:
    """Median, minimum and maximum microseconds per launch of `launch(i)`
    (i = running launch index, which picks the buffer set) over `samples`
    batches of back-to-back launches, each at least `sample_ms` long, after
    at least `warmup_ms` of warm-up launches.  Each batch starts with a few
    untimed launches, so that the GPU is busy when the start event is
    reached and no host-side gap enters the batch."""
    i = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < warmup_ms:
        for _ in range(min(64, calib)):
            launch(i)
            i += 1
        torch.cuda.synchronize()
    # launches per batch from a short calibration batch
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(calib):
        launch(i)
        i += 1
    z.record(stream)
    torch.cuda.synchronize()
    est_us = a.elapsed_time(z) * 1e3 / calib
    n = max(calib, int(sample_ms * 1e3 / est_us * 1.1) + 1)
    vals = []
    for _ in range(samples):
        for _ in range(8):
            launch(i)
            i += 1
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            launch(i)
            i += 1
        z.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(z)
        vals.append(ms * 1e3 / n)
    vals.sort()
    return {"median": vals[len(vals) // 2], "min": vals[0], "max": vals[-1], "launches_per_sample": n,
            "sample_ms": round(vals[len(vals) // 2] * n / 1e3, 2)}


def trace_fraction(lr, op: str, nbytes: int) -> dict:
    """The kernel-trace average duration of `op`'s kernel instance from the
    committed rocprofv3 summary, and the roofline fraction it gives; nulls
    when the kernels changed since the trace was taken or the summary holds
    another instance than this plan launches."""
    from row_reductions_amd import profiling
    plan = lr.lr_plan_query(op, ROWS, COLS, "unordered_tree")
    params = {"softmax": 0, "rmsnorm": 1, "layernorm": 1}[op]
    kernel = profiling.kernel_name(lr.OPS[op], plan, True, params)
    rec = profiling.lookup(TRACE_SUMMARY, op, kernel)
    if rec is None:
        return {"trace_us": None, "frac_trace": None}
    return {"trace_us": round(rec["avg_us"], 3), "frac_trace": round(nbytes / (rec["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "trace_dispatches": rec["dispatches"]}


def device_record(lr, torch) -> dict:
    """The device the figures were taken on: its name, compute units, and the
    memory clock and bus width the runtime reports.  The fractions divide by
    the published 8 TB/s; over the reported bus that is the per-pin rate
    given here (HBM3E moves several bits per pin per reported clock)."""
    props = torch.cuda.get_device_properties(0)
    rec = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
           "compute_units": props.multi_processor_count, "hbm_peak_used_gbs": HBM_PEAK_GBS}
    try:
        clk_khz, bus_bits = lr.lr_device_memory_query()
    except lr.LrError:
        return rec
    rec.update({"memory_clock_khz": clk_khz, "memory_bus_bits": bus_bits})
    if bus_bits > 0 and clk_khz > 0:
        gbps_per_pin = HBM_PEAK_GBS * 8 / bus_bits
        rec.update({"peak_per_pin_gbps": round(gbps_per_pin, 3),
                    "peak_transfers_per_reported_clock": round(gbps_per_pin * 1e9 / (clk_khz * 1e3), 3)})
    return rec


def op_bytes(rows: int, cols: int) -> int:
    """Algorithmic bytes of one softmax / norm launch: read + write of the tensor."""
    return 2 * rows * cols * 4


def ce_bytes(rows: int, cols: int) -> int:
    """Cross-entropy: logits read, int64 labels read, FP32 losses written."""
    return rows * cols * 4 + rows * 8 + rows * 4


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--sets", type=int, default=32, help="rotating buffer sets per op (cold cache)")
    ap.add_argument("--warm", action="store_true", help="time one buffer set (cache-warm) as the main figure")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU work budget of the oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the warm and cross-entropy context figures")
    ap.add_argument("--samples", type=int, default=SAMPLES, help="per-op protocol: batches per op")
    ap.add_argument("--sample-ms", type=float, default=SAMPLE_MS, help="per-op protocol: least duration of a batch")
    ap.add_argument("--warmup-ms", type=float, default=WARMUP_MS, help="per-op protocol: least warm-up")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also launch a plain device copy of known size (counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the row-reduction path has no multi-GPU part "
              "(rows are independent: G GPUs would each run the same kernels on rows / G rows, "
              "with no exchange).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import row_reductions_amd as lr
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    # ---------------- inputs (seeded, device-resident) ----------------
    soft = synth.softmax_inputs(ROWS, COLS, seed=0)
    rms = synth.rmsnorm_inputs(ROWS, COLS, seed=0)
    ln = synth.layernorm_inputs(ROWS, COLS, seed=0)
    nsets = 1 if args.warm else args.sets

    def device_sets(x: np.ndarray):
        xt = torch.from_numpy(x).to(dev)
        xs = [xt] + [xt.clone() for _ in range(nsets - 1)]
        ys = [torch.empty_like(xt) for _ in range(nsets)]
        return xs, ys

    sx, sy = device_sets(soft["x"])
    rx, ry = device_sets(rms["x"])
    lx, ly = device_sets(ln["x"])
    rg = torch.from_numpy(rms["gamma"]).to(dev)
    lg = torch.from_numpy(ln["gamma"]).to(dev)
    lb = torch.from_numpy(ln["beta"]).to(dev)

    def launch(op: str, i: int, policy: int = lr.LR_UNORDERED_TREE) -> None:
        k = i % nsets
        if op == "softmax":
            st = lr.lib.lr_softmax_f32(sx[k].data_ptr(), sy[k].data_ptr(), ROWS, COLS, policy, sh)
        elif op == "rmsnorm":
            st = lr.lib.lr_rmsnorm_f32(rx[k].data_ptr(), rg.data_ptr(), ry[k].data_ptr(), ROWS, COLS,
                                       EPS["rmsnorm"], policy, sh)
        else:
            st = lr.lib.lr_layernorm_f32(lx[k].data_ptr(), lg.data_ptr(), lb.data_ptr(), ly[k].data_ptr(),
                                         ROWS, COLS, EPS["layernorm"], policy, sh)
        if st != 0:
            raise lr.LrError(st, op)

    # ---------------- warmup ----------------
    for i in range(args.warmup):
        for op in OPS:
            launch(op, i)
    torch.cuda.synchronize()

    # ---------------- timed region: K steps ----------------
    # events only at the edges: a marker between kernels would serialise the
    # stream and add its own gap to every launch
    K = args.steps
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for i in range(K):
        for op in OPS:
            launch(op, i)
    t_end.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    gpu_ms_per_step = t_start.elapsed_time(t_end) / K

    # per-op launch duration: each op alone, the pages' protocol (warm-up of
    # at least 200 ms, nine batches of at least 30 ms, median and range)
    progress(f"timed {K} steps: {ms_per_step * 1e3:.2f} us per step")
    per_op = {}
    for op in OPS:
        per_op[op] = time_batches(torch, stream, lambda i, op=op: launch(op, i), samples=args.samples,
                                  sample_ms=args.sample_ms, warmup_ms=args.warmup_ms)
        progress(f"{op}: {per_op[op]['median']:.3f} us per launch (median of {args.samples} batches)")
    per_op_us = {op: per_op[op]["median"] for op in OPS}

    b = op_bytes(ROWS, COLS)
    step_bytes = b * len(OPS)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    gbps = {op: b / (per_op_us[op] * 1e-6) / 1e9 for op in OPS}
    dominant = max(OPS, key=lambda o: per_op_us[o])
    achieved = gbps[dominant]

    # single-call latency: one launch between synchronisations
    single = {}
    for op in OPS:
        vals = []
        for i in range(20):
            torch.cuda.synchronize()
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            launch(op, i)
            z.record(stream)
            torch.cuda.synchronize()
            vals.append(a.elapsed_time(z) * 1e3)
        single[op] = float(np.median(vals))

    plans = {}
    for op in OPS:
        p = lr.lr_plan_query(op, ROWS, COLS, "unordered_tree")
        plans[op] = {k: v for k, v in p.as_dict().items() if k in (
            "family", "waves_per_row", "rows_per_block", "chunks_per_lane", "threads_per_block", "blocks")}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "gpu_ms_per_step": round(gpu_ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / (step_bytes / (PAGES_M1MAX_STEP_US * 1e-6) / 1e9), 3),
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "softmax + RMSNorm + LayerNorm, FP32 768x6144 each (x~N(0,1), gamma~U(0.5,1.5), "
                        "beta~N(0,0.1^2), eps 1e-6/1e-5), unordered_tree",
            "rows": ROWS, "cols": COLS, "ops": list(OPS), "policy": "unordered_tree",
            "cache_state": ("warm (one buffer set)" if args.warm else
                            f"cold ({nsets} rotating buffer sets per op, "
                            f"{nsets * b * len(OPS) / 1e9:.2f} GB)"),
            "bytes_per_step": step_bytes,
            "vs_baseline_note": "ratio to the pages' Apple M1 Max command-buffer medians "
                                "(57.414/60.753/75.251 us); context, not a target",
        },
        "us_per_op": {op: round(per_op_us[op], 3) for op in OPS},
        "us_per_op_range": {op: [round(per_op[op]["min"], 3), round(per_op[op]["max"], 3)] for op in OPS},
        "per_op_protocol": (f"median of {args.samples} batches of >= {args.sample_ms:g} ms of back-to-back cold "
                            f"launches ({per_op[OPS[0]]['launches_per_sample']} launches of {OPS[0]} per batch) "
                            f"after >= {args.warmup_ms:g} ms of warm-up, HIP events on the launch stream"),
        "single_call_us": single,
        "gbps_per_op": {op: round(gbps[op], 1) for op in OPS},
        "pct_of_hbm_peak_per_op": {op: round(100 * gbps[op] / HBM_PEAK_GBS, 2) for op in OPS},
        "plans": plans,
        "device": device_record(lr, torch),
        "roofline": {
            "kernel": dominant,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_bytes(lr, dominant),
            "bytes_per_launch": b,
            "avg_launch_us": round(per_op_us[dominant], 3),
            "avg_launch_us_range": [round(per_op[dominant]["min"], 3), round(per_op[dominant]["max"], 3)],
            "gate": "frac (back-to-back launches, event-timed median); frac_trace is the kernel-trace duration "
                    "of the committed rocprofv3 profile, where every dispatch starts on an idle GPU",
            **trace_fraction(lr, dominant, b),
        },
    }

    # ---------------- context: warm cache and cross-entropy ----------------
    if not args.no_extra:
        extra = {}
        if not args.warm:
            for op in OPS:
                t = time_batches(torch, stream, lambda i, op=op: launch(op, 0), samples=5)
                extra[f"{op}_768x6144_warm"] = {"us_per_op": round(t["median"], 3),
                                                "range": [round(t["min"], 3), round(t["max"], 3)],
                                                "gbps": round(b / t["median"] / 1e3, 1)}
        # the deterministic policies on the same step (cold)
        for pol, pname in ((lr.LR_ORDERED_TREE, "ordered_tree"), (lr.LR_ORDERED_FOLD, "ordered_fold"),
                           (lr.LR_FOLD_RIGHT, "fold_right")):
            for op in OPS:
                t = time_batches(torch, stream, lambda i, op=op, pol=pol: launch(op, i, pol), samples=5)
                extra[f"{op}_768x6144_{pname}_cold"] = {"us_per_op": round(t["median"], 3),
                                                        "range": [round(t["min"], 3), round(t["max"], 3)],
                                                        "gbps": round(b / t["median"] / 1e3, 1)}
        # the norms called without their parameters (cold): a plan of their own
        for op in ("rmsnorm", "layernorm"):
            def bare(i, op=op):
                k = i % nsets
                if op == "rmsnorm":
                    st = lr.lib.lr_rmsnorm_f32(rx[k].data_ptr(), None, ry[k].data_ptr(), ROWS, COLS,
                                               EPS["rmsnorm"], lr.LR_UNORDERED_TREE, sh)
                else:
                    st = lr.lib.lr_layernorm_f32(lx[k].data_ptr(), None, None, ly[k].data_ptr(), ROWS, COLS,
                                                 EPS["layernorm"], lr.LR_UNORDERED_TREE, sh)
                if st != 0:
                    raise lr.LrError(st, op)
            t = time_batches(torch, stream, bare, samples=5)
            extra[f"{op}_768x6144_no_params_cold"] = {"us_per_op": round(t["median"], 3),
                                                      "range": [round(t["min"], 3), round(t["max"], 3)],
                                                      "gbps": round(b / t["median"] / 1e3, 1)}
        progress("warm-cache and ordered-policy figures done")
        extra.update(add_layernorm_extra(lr, synth, torch, dev, sh, stream, nsets))
        extra.update(small_configs_graph(lr, synth, torch, dev))
        progress("fused residual LayerNorm and launch-bound workloads done")
        ce = synth.cross_entropy_inputs(4096, 32000, seed=0)
        cx = [torch.from_numpy(ce["logits"]).to(dev)]
        cx.append(cx[0].clone())
        clab = torch.from_numpy(ce["labels"]).to(dev)
        closs = torch.empty(4096, device=dev)
        del ce
        for i in range(4):
            lr.check(lr.lib.lr_cross_entropy_f32(cx[i % 2].data_ptr(), clab.data_ptr(), closs.data_ptr(),
                                                 4096, 32000, 0, sh))
        t = time_batches(torch, stream, lambda i: lr.lib.lr_cross_entropy_f32(
            cx[i % 2].data_ptr(), clab.data_ptr(), closs.data_ptr(), 4096, 32000, 0, sh), samples=5)
        us = t["median"]
        cb = ce_bytes(4096, 32000)
        p = lr.lr_plan_query("cross_entropy", 4096, 32000)
        extra["cross_entropy_4096x32000_cold"] = {
            "us_per_op": round(us, 3), "range": [round(t["min"], 3), round(t["max"], 3)],
            "gbps": round(cb / us / 1e3, 1),
            "pct_of_hbm_peak": round(100 * cb / us / 1e3 / HBM_PEAK_GBS, 2), "bytes": cb,
            "plan": {k: v for k, v in p.as_dict().items() if k in (
                "family", "waves_per_row", "rows_per_block", "chunks_per_lane", "threads_per_block")}}
        # row sum and row minimum/maximum over the same logits (read-only ops)
        rsum = torch.empty(4096, device=dev)
        rmin, rmax = torch.empty(4096, device=dev), torch.empty(4096, device=dev)
        for name, fn, outb in (
            ("row_sum_4096x32000_cold",
             lambda i: lr.lib.lr_row_sum_f32(cx[i % 2].data_ptr(), rsum.data_ptr(), 4096, 32000, 0, sh), 4),
            ("row_minmax_4096x32000_cold",
             lambda i: lr.lib.lr_row_minmax_f32(cx[i % 2].data_ptr(), rmin.data_ptr(), rmax.data_ptr(), 4096,
                                                32000, 0, sh), 8)):
            for i in range(4):
                lr.check(fn(i), name)
            t = time_batches(torch, stream, fn, samples=5)
            us = t["median"]
            rb = 4096 * 32000 * 4 + 4096 * outb
            extra[name] = {"us_per_op": round(us, 3), "range": [round(t["min"], 3), round(t["max"], 3)],
                           "gbps": round(rb / us / 1e3, 1),
                           "pct_of_hbm_peak": round(100 * rb / us / 1e3 / HBM_PEAK_GBS, 2), "bytes": rb}
        del cx
        # narrow rows (several rows per wave): 262144 x 64, four rotating
        # 67 MB input/output sets (537 MB, past the Infinity Cache)
        nx = [torch.randn(262144, 64, device=dev) for _ in range(4)]
        ny = [torch.empty_like(t) for t in nx]
        ng, nb = torch.rand(64, device=dev) + 0.5, torch.randn(64, device=dev) * 0.1
        for name, op, pol, fn in (
            ("softmax_262144x64_cold", "softmax", 0,
             lambda i: lr.lib.lr_softmax_f32(nx[i % 4].data_ptr(), ny[i % 4].data_ptr(), 262144, 64, 0, sh)),
            ("layernorm_262144x64_cold", "layernorm", 0,
             lambda i: lr.lib.lr_layernorm_f32(nx[i % 4].data_ptr(), ng.data_ptr(), nb.data_ptr(),
                                               ny[i % 4].data_ptr(), 262144, 64, 1e-5, 0, sh)),
            # the ordered fold with one lane per row
            ("rmsnorm_262144x64_ordered_fold_cold", "rmsnorm", 1,
             lambda i: lr.lib.lr_rmsnorm_f32(nx[i % 4].data_ptr(), ng.data_ptr(), ny[i % 4].data_ptr(), 262144, 64,
                                             1e-6, 1, sh))):
            for i in range(8):
                lr.check(fn(i), name)
            t = time_batches(torch, stream, fn, samples=5)
            us = t["median"]
            nbytes = op_bytes(262144, 64)
            p = lr.lr_plan_query(op, 262144, 64, pol)
            extra[name] = {"us_per_op": round(us, 3), "range": [round(t["min"], 3), round(t["max"], 3)],
                           "gbps": round(nbytes / us / 1e3, 1),
                           "pct_of_hbm_peak": round(100 * nbytes / us / 1e3 / HBM_PEAK_GBS, 2), "bytes": nbytes,
                           "plan": {k: v for k, v in p.as_dict().items() if k in (
                               "family", "lanes_per_row", "rows_per_block", "chunks_per_lane", "threads_per_block")}}
        del nx, ny
        out["extra"] = extra

    if args.copy_probe:
        # plain device-to-device copies of one 768x6144 tensor: the reference
        # kernel for scaling FETCH_SIZE / WRITE_SIZE counters to bytes
        for _ in range(20):
            sy[0].copy_(sx[0])
        torch.cuda.synchronize()

    # ---------------- CPU baseline: the oracle on the host cores ----------------
    if not args.no_cpu_baseline:
        progress("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(soft, rms, ln, args.cpu_seconds)

    print(json.dumps(out), flush=True)


def small_configs_graph(lr, synth, torch, dev) -> dict:
    """The launch-bound workloads (softmax 37x1537, RMSNorm 256x3072 under both
    listed policies, LayerNorm 64x12289 without and with a workspace for the
    split-row kernels): 200 launches captured in one HIP
    graph and replayed, so the per-launch time is the GPU's, not the host's
    launch rate.  Inputs stay resident (one buffer set: these tensors fit in
    the L2s, as they do between a producer and this kernel in practice)."""
    out = {}
    n = 200
    cases = []
    sx = torch.from_numpy(synth.workload_inputs("softmax_37x1537")["x"]).to(dev)
    sy = torch.empty_like(sx)
    cases.append(("softmax_37x1537", lambda sh: lr.lr_softmax_f32(sx, sy, 37, 1537, 0, sh), 2 * sx.numel() * 4))
    rin = synth.workload_inputs("rmsnorm_256x3072")
    rx, rg = torch.from_numpy(rin["x"]).to(dev), torch.from_numpy(rin["gamma"]).to(dev)
    ry = torch.empty_like(rx)
    for pol, name in ((0, "unordered_tree"), (1, "ordered_fold"), (2, "ordered_tree")):
        cases.append((f"rmsnorm_256x3072_{name}",
                      lambda sh, pol=pol: lr.lr_rmsnorm_f32(rx, rg, ry, 256, 3072, 1e-6, pol, sh), 2 * rx.numel() * 4))
    lin = synth.workload_inputs("layernorm_64x12289")
    lx = torch.from_numpy(lin["x"]).to(dev)
    lg, lb = torch.from_numpy(lin["gamma"]).to(dev), torch.from_numpy(lin["beta"]).to(dev)
    ly = torch.empty_like(lx)
    cases.append(("layernorm_64x12289", lambda sh: lr.lr_layernorm_f32(lx, lg, lb, ly, 64, 12289, 1e-5, 0, sh),
                  2 * lx.numel() * 4))
    # the same with rows split across workgroups through a workspace (two
    # kernels; the fastest split plan, given explicitly: the planner keeps
    # one launch here, which is faster)
    sp = next(p for p in lr.lr_plan_enumerate(lr.lr_device_facts_query(), "layernorm", 64, 12289, "unordered_tree", 0)
              if p.family == lr.LR_FAMILY_SPLIT and p.splits == 4 and p.waves_per_row == 8 and p.chunks_per_lane == 2)
    lws = torch.empty(lr.lr_plan_workspace_bytes(sp, 64), dtype=torch.uint8, device=dev)
    cases.append(("layernorm_64x12289_split",
                  lambda sh: lr.lr_layernorm_f32(lx, lg, lb, ly, 64, 12289, 1e-5, 0, sh, plan=sp, workspace=lws),
                  2 * lx.numel() * 4))
    for name, fn, nbytes in cases:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            lr.check(fn(side.cuda_stream), name)  # warm the plan cache outside the capture
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=side):
                for _ in range(n):
                    fn(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        # one "launch" of the protocol is one replay of n kernels
        t = time_batches(torch, torch.cuda.current_stream(), lambda i: graph.replay(), samples=5, calib=8)
        us = t["median"] / n
        out[f"{name}_graph"] = {"us_per_op": round(us, 3), "range": [round(t["min"] / n, 3), round(t["max"] / n, 3)],
                                "gbps": round(nbytes / us / 1e3, 1)}
    return out


def add_layernorm_extra(lr, synth, torch, dev, sh, stream, nsets) -> dict:
    """Fused residual LayerNorm 768x6144 (x, residual, gamma, beta in; y out,
    with and without the combined output), rotating buffer sets as the step."""
    inp = synth.add_layernorm_inputs(ROWS, COLS, seed=0)
    x0 = torch.from_numpy(inp["x"]).to(dev)
    r0 = torch.from_numpy(inp["residual"]).to(dev)
    xs = [x0] + [x0.clone() for _ in range(nsets - 1)]
    rs = [r0] + [r0.clone() for _ in range(nsets - 1)]
    ys = [torch.empty_like(x0) for _ in range(nsets)]
    ss = [torch.empty_like(x0) for _ in range(nsets)]
    g = torch.from_numpy(inp["gamma"]).to(dev)
    b = torch.from_numpy(inp["beta"]).to(dev)
    out = {}
    tb = ROWS * COLS * 4
    for with_sum in (False, True):
        def launch(i):
            k = i % nsets
            st = lr.lib.lr_add_layernorm_f32(xs[k].data_ptr(), rs[k].data_ptr(), g.data_ptr(), b.data_ptr(),
                                             ys[k].data_ptr(), ss[k].data_ptr() if with_sum else None,
                                             ROWS, COLS, EPS["layernorm"], 0, sh)
            if st != 0:
                raise lr.LrError(st, "add_layernorm")
        t = time_batches(torch, stream, launch, samples=5)
        us = t["median"]
        moved = (4 if with_sum else 3) * tb
        key = "add_layernorm_768x6144_cold" + ("_with_sum" if with_sum else "")
        out[key] = {"us_per_op": round(us, 3), "range": [round(t["min"], 3), round(t["max"], 3)],
                    "gbps": round(moved / us / 1e3, 1),
                    "pct_of_hbm_peak": round(100 * moved / us / 1e3 / HBM_PEAK_GBS, 2), "bytes": moved}
    del xs, rs, ys, ss
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.machine()


def cpu_baseline(soft, rms, ln, budget_s: float) -> dict:
    """The double-precision oracle, unmodified, on the same 768x6144 inputs,
    timed two ways: rows split over the host threads this process may use
    (at most 16, the CPU share of one GPU; the C oracle releases the GIL),
    the whole three-op workload repeated until `budget_s` seconds are used;
    and on one thread over the first 96 rows of each op for up to
    budget_s / 2 seconds, scaled to the same GB/s unit."""
    import concurrent.futures as cf

    import numpy as np

    import oracle

    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    cores = max(1, min(16, avail))
    chunks = np.array_split(np.arange(ROWS), cores)

    def run_rows(lo, hi):
        oracle.softmax(soft["x"][lo:hi])
        oracle.rmsnorm(rms["x"][lo:hi], rms["gamma"], EPS["rmsnorm"])
        oracle.layernorm(ln["x"][lo:hi], ln["gamma"], ln["beta"], EPS["layernorm"])

    reps = 0
    with cf.ThreadPoolExecutor(max_workers=cores) as ex:
        t0 = time.perf_counter()
        while True:
            list(ex.map(lambda idx: run_rows(int(idx[0]), int(idx[-1]) + 1), chunks))
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 1000:
                break
    step_s = el / reps
    step_bytes = op_bytes(ROWS, COLS) * len(OPS)

    # one thread, a bounded sample: the first 96 rows of each op
    srows = 96
    reps1 = 0
    t0 = time.perf_counter()
    while True:
        run_rows(0, srows)
        reps1 += 1
        el1 = time.perf_counter() - t0
        if el1 >= budget_s / 2 or reps1 >= 1000:
            break
    one_s = el1 / reps1
    one_bytes = op_bytes(srows, COLS) * len(OPS)
    return {
        "value": round(step_bytes / step_s / 1e9, 3),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"full workload (softmax+RMSNorm+LayerNorm 768x6144), {reps} repetitions in {el:.1f} s, "
                  f"rows split over {cores} threads; {step_s * 1e3:.2f} ms per step",
        "single_thread": {"value": round(one_bytes / one_s / 1e9, 3), "unit": "GB/s", "cores": 1,
                          "sample": f"first {srows} rows of each op, {reps1} repetitions in {el1:.1f} s; "
                                    f"{one_s * 1e3 * ROWS / srows:.1f} ms per full step (scaled)"},
        "nproc": os.cpu_count(),
        "affinity_cores": avail,
        "cpu": _cpu_model(),
    }


if __name__ == "__main__":
    main()
