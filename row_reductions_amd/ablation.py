"""Cache / reload x stripe width ablation at 768 x 6144 (softmax, RMSNorm,
LayerNorm), with the register count and occupancy of every plan.

Plans: the CACHE family at every S = 1..16 waves per row (the smallest
compiled chunk count that covers the row: the register stripe narrows as S
grows) and the STREAM family (no register copy; passes reload the row) at
S = 1, 2, 4, 8, 16; one row per workgroup.  Each plan is timed as a batch of
back-to-back cold launches (32 rotating buffer sets) between two HIP events.

    python -m row_reductions_amd.ablation run --out R.jsonl
    rocprofv3 --pmc OccupancyPercent --output-format csv -d D -o run -- \\
        python -m row_reductions_amd.ablation run --iters 40
    python -m row_reductions_amd.ablation summarize --results R.jsonl \\
        --counters D/run_counter_collection.csv --out profiles/ablation_768x6144.md

The counter run gives, per dispatch, the VGPRs the kernel was allocated,
its scratch (spill) size and rocprofv3's OccupancyPercent (resident wave
cycles over the device's wave slots while the GPU is busy).
"""
from __future__ import annotations

import argparse
import csv
import json
import re
import sys
from collections import defaultdict

ROWS, COLS = 768, 6144
OPS = ("softmax", "rmsnorm", "layernorm")
STREAM_S = (1, 2, 4, 8, 16)
TENSOR_BYTES = ROWS * COLS * 4


def plans(lr, op):
    facts = lr.lr_device_facts_mi355x()
    out = []
    for p in lr.lr_plan_enumerate(facts, op, ROWS, COLS, "unordered_tree", 1):
        if p.rows_per_block != 1:
            continue
        if p.family == lr.LR_FAMILY_CACHE or (p.family == lr.LR_FAMILY_STREAM and p.waves_per_row in STREAM_S):
            out.append(p)
    return out


def run(args) -> int:
    import torch

    import row_reductions_amd as lr
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    gen = torch.Generator(device=dev).manual_seed(0)
    x0 = torch.randn(ROWS, COLS, device=dev, generator=gen)
    xs = [x0] + [x0.clone() for _ in range(args.sets - 1)]
    ys = [torch.empty_like(x0) for _ in range(args.sets)]
    g = torch.rand(COLS, device=dev, generator=gen) + 0.5
    b = torch.randn(COLS, device=dev, generator=gen) * 0.1
    out = open(args.out, "w") if args.out else sys.stdout

    def launcher(op, p):
        def f(i):
            k = i % args.sets
            if op == "softmax":
                return lr.lr_softmax_f32(xs[k], ys[k], ROWS, COLS, 0, sh, p)
            if op == "rmsnorm":
                return lr.lr_rmsnorm_f32(xs[k], g, ys[k], ROWS, COLS, 1e-6, 0, sh, p)
            return lr.lr_layernorm_f32(xs[k], g, b, ys[k], ROWS, COLS, 1e-5, 0, sh, p)
        return f

    for op in OPS:
        for p in plans(lr, op):
            f = launcher(op, p)
            for i in range(10):
                lr.check(f(i), op)
            torch.cuda.synchronize()
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(args.iters):
                f(i)
            z.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(z) * 1e3 / args.iters
            rec = dict(op=op, family=lr.FAMILY_NAMES[p.family], S=p.waves_per_row, nch=p.chunks_per_lane,
                       threads=p.threads_per_block, us=round(us, 3),
                       gbps=round(2 * TENSOR_BYTES / us / 1e3, 1))
            print(json.dumps(rec), file=out, flush=True)
    return 0


_KNAME = re.compile(r"lr::k_(cache|stream)<(\d+), (?:(\d+), )?(true|false)")


def summarize(args) -> int:
    results = [json.loads(line) for line in open(args.results) if line.startswith("{")]
    occ = defaultdict(list)
    res = {}
    with open(args.counters) as f:
        for r in csv.DictReader(f):
            m = _KNAME.search(r["Kernel_Name"])
            if not m or m.group(4) != "true":
                continue
            fam, op = m.group(1), OPS[int(m.group(2))] if int(m.group(2)) < 3 else None
            if op is None:
                continue
            nch = int(m.group(3)) if m.group(3) else 4
            key = (op, fam, int(r["Workgroup_Size"]) // 64, nch)
            occ[key].append(float(r["Counter_Value"]))
            res[key] = (int(r["VGPR_Count"]), int(r["Scratch_Size"]))
    lines = [
        "# Cache / reload x stripe width ablation, FP32 768x6144 (MI355X, cold)",
        "",
        "Commands (repository root, GPU box, `TMPDIR=/tmp`):",
        "",
        "```",
        "python -m row_reductions_amd.ablation run --out gpurun_out/ablation.jsonl",
        "rocprofv3 --pmc OccupancyPercent --output-format csv -d gpurun_out/occ -o run -- \\",
        "    python -m row_reductions_amd.ablation run --iters 40",
        "python -m row_reductions_amd.ablation summarize --results gpurun_out/ablation.jsonl \\",
        "    --counters gpurun_out/occ/run_counter_collection.csv --out profiles/ablation_768x6144.md",
        "```",
        "",
        "One row per workgroup.  CACHE keeps the row's stripe in registers (chunks per lane = the",
        "smallest compiled instance covering 1536 chunks over 64*S lanes); STREAM reloads the row",
        "for each pass (softmax 2 reads, RMSNorm 2, LayerNorm 3).  `us` is the HIP-event average of",
        f"a batch of back-to-back launches over 32 rotating buffer sets; GB/s counts {2 * TENSOR_BYTES:,} B",
        "per launch (tensor read + write).  VGPRs and scratch are what the dispatch was allocated",
        "(rocprofv3); occupancy is rocprofv3's OccupancyPercent, the mean over the counter run's",
        "dispatches of resident wave cycles against the device's wave slots while it is busy.",
        "",
    ]
    for op in OPS:
        lines += [f"## {op}", "", "| family | S | chunks/lane | VGPRs | scratch | occupancy % | us | GB/s |",
                  "|---|---:|---:|---:|---:|---:|---:|---:|"]
        rows = [r for r in results if r["op"] == op]
        best = min(r["us"] for r in rows)
        for r in sorted(rows, key=lambda r: (r["family"], r["S"])):
            key = (op, r["family"], r["S"], r["nch"])
            vgprs, scratch = res.get(key, ("-", "-"))
            o = occ.get(key)
            occupancy = f"{sum(o) / len(o):.1f}" if o else "-"
            mark = " **(best)**" if r["us"] == best else ""
            lines.append(f"| {r['family']} | {r['S']} | {r['nch']} | {vgprs} | {scratch} | {occupancy} | "
                         f"{r['us']:.2f}{mark} | {r['gbps']:.0f} |")
        lines.append("")
    open(args.out, "w").write("\n".join(lines))
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--iters", type=int, default=300)
    r.add_argument("--sets", type=int, default=32)
    r.add_argument("--out", default="")
    s = sub.add_parser("summarize")
    s.add_argument("--results", required=True)
    s.add_argument("--counters", required=True)
    s.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    return run(args) if args.cmd == "run" else summarize(args)


if __name__ == "__main__":
    sys.exit(main())
