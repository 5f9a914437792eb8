"""Measured plan selection for one problem shape (staged tuning).

Follows the authority split of "TIRx Metal reduction lowering", section 7:
legality comes from the planner (every candidate is a legal plan of
lr_plan_enumerate), and the fastest *valid* candidate, measured on the
device, is the winner.  Each candidate's output is checked against the
automatic plan's output (|a - b| <= 1e-6 + 1e-5 |b|); a candidate that fails
is reported and never selected.  The winner is re-measured before it is
printed as a line for lr_plan_table.inc.

    python -m row_reductions_amd.tune --op layernorm --rows 768 --cols 6144

Timing: `--sets` rotating input/output buffer sets (cold cache by default),
`--iters` back-to-back launches on one stream between two HIP events.  With
`--graph` the `--iters` launches are captured in one HIP graph and replayed
(three replays between the events): the per-launch time is then the GPU's
and not the host's launch rate, which bounds eager calls near 4 us, so this
is the mode for launch-bound shapes.
"""
from __future__ import annotations

import argparse
import json
import sys

import torch

import row_reductions_amd as lr


def _launcher(op, xs, ys, g, b, lab, rows, cols, eps, policy, sh, rs=None, ys2=None, ws=None):
    """run(i, plan): one launch on buffer set i; split plans use workspace ws."""
    pol = lr._policy(policy)

    def run(i, plan, stream=None):
        sh_ = sh if stream is None else stream
        k = i % len(xs)
        w = ws if plan is not None and plan.family == lr.LR_FAMILY_SPLIT else None
        if op == "softmax":
            return lr.lr_softmax_f32(xs[k], ys[k], rows, cols, pol, sh_, plan, workspace=w)
        if op == "rmsnorm":
            return lr.lr_rmsnorm_f32(xs[k], g, ys[k], rows, cols, eps, pol, sh_, plan, workspace=w)
        if op == "layernorm":
            return lr.lr_layernorm_f32(xs[k], g, b, ys[k], rows, cols, eps, pol, sh_, plan, workspace=w)
        if op == "add_layernorm":
            return lr.lr_add_layernorm_f32(xs[k], rs[k], g, b, ys[k], None, rows, cols, eps, pol, sh_, plan,
                                           workspace=w)
        if op == "row_sum":
            return lr.lr_row_sum_f32(xs[k], ys[k], rows, cols, pol, sh_, plan, workspace=w)
        if op == "row_minmax":
            return lr.lr_row_minmax_f32(xs[k], ys[k], ys2[k], rows, cols, pol, sh_, plan, workspace=w)
        return lr.lr_cross_entropy_f32(xs[k], lab, ys[k], rows, cols, pol, sh_, plan, workspace=w)
    return run


def _time(run, plan, iters, stream):
    for i in range(5):
        lr.check(run(i, plan), "warmup")
    torch.cuda.synchronize()
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(iters):
        run(i, plan)
    z.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(z) * 1e3 / iters


def _time_graph(run, plan, iters, stream, reps=3):
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        lr.check(run(0, plan, side.cuda_stream), "warmup")
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            for i in range(iters):
                run(i, plan, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        graph.replay()
    z.record(stream)
    torch.cuda.synchronize()
    del graph
    return a.elapsed_time(z) * 1e3 / (iters * reps)


def _parse_plan(spec, enum, auto):
    if spec == "auto":
        return auto
    f = spec.split(":")
    fam = {name: code for code, name in lr.FAMILY_NAMES.items()}[f[0]]
    S, Q, nch = map(int, f[1:4])
    n = int(f[4]) if len(f) > 4 else 0
    splits = n if fam == lr.LR_FAMILY_SPLIT else 0
    lanes = n if fam == lr.LR_FAMILY_CACHE and n else 64 * S
    for p in enum:
        if (p.family, p.waves_per_row, p.rows_per_block, p.chunks_per_lane, p.splits, p.lanes_per_row) == \
                (fam, S, Q, nch, splits, lanes):
            return p
    raise SystemExit(f"{spec}: not a legal plan of this problem")


def _compare(args, op, rows, cols, aligned, facts, auto, run, ys, ref, bound, timer, stream):
    """A/B of explicit plans: each round times every plan once, in alternating
    order; medians (and minima) over the rounds."""
    enum = lr.lr_plan_enumerate(facts, op, rows, cols, args.policy, aligned)
    plans = [(spec, _parse_plan(spec, enum, auto)) for spec in args.compare]
    for spec, p in plans:
        st = run(0, p)
        torch.cuda.synchronize()
        if st != lr.LR_OK or not bool(((ys[0].double() - ref).abs() <= bound).all()):
            raise SystemExit(f"{spec}: output differs from the automatic plan's")
    times = {spec: [] for spec, _ in plans}
    for r in range(args.rounds):
        for spec, p in (plans if r % 2 == 0 else plans[::-1]):
            times[spec].append(timer(run, p, args.iters, stream))
    mode = "graph" if args.graph else "eager"
    print(f"# {op} {rows}x{cols} {args.policy} ({mode}), A/B over {args.rounds} rounds: median us (min)")
    for spec, p in plans:
        v = sorted(times[spec])
        print(f"#   {spec:22s} {v[len(v) // 2]:8.3f} ({v[0]:.3f})  {p!r}")
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description="exhaustive measured plan sweep for one shape")
    ap.add_argument("--op", required=True, choices=sorted(lr.OPS))
    ap.add_argument("--rows", type=int, required=True)
    ap.add_argument("--cols", type=int, required=True)
    ap.add_argument("--policy", default="unordered_tree", choices=sorted(lr.POLICIES))
    ap.add_argument("--eps", type=float, default=1e-5)
    ap.add_argument("--sets", type=int, default=0, help="rotating buffer sets (0: enough for >= 1 GB)")
    ap.add_argument("--iters", type=int, default=200)
    ap.add_argument("--max-rows-per-block", type=int, default=4,
                    help="whole-wave plans: rows per workgroup; sub-wave plans: waves per workgroup")
    ap.add_argument("--json", action="store_true", help="one JSON line per candidate")
    ap.add_argument("--graph", action="store_true", help="time HIP-graph replays (launch-bound shapes)")
    ap.add_argument("--compare", nargs="+", metavar="PLAN",
                    help="instead of the sweep: A/B of the given plans, alternating for --rounds rounds; "
                         "PLAN is 'auto' (the typed entry points' plan) or family:S:Q:chunks[:N], "
                         "family one of cache, stream, ordered, tree, split; N is the split count of a "
                         "split plan, the lanes per row of a sub-wave cache plan")
    ap.add_argument("--rounds", type=int, default=6)
    ap.add_argument("--no-params", action="store_true",
                    help="RMSNorm / LayerNorm called without gamma and beta ('auto' is then the typed call's "
                         "plan, which may be one listed for that case)")
    args = ap.parse_args(argv)
    if args.no_params and args.op not in ("rmsnorm", "layernorm", "add_layernorm"):
        raise SystemExit("--no-params applies to the norms")

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    rows, cols, op = args.rows, args.cols, args.op
    tensor_bytes = rows * cols * 4
    sets = args.sets or max(2, min(64, -(-(1 << 30) // (2 * tensor_bytes))))
    gen = torch.Generator(device=dev).manual_seed(0)
    x0 = torch.randn(rows, cols, device=dev, generator=gen)
    if op == "row_sum":
        x0 = x0.abs()  # positive rows: sums of any order agree to the relative bar
    xs = [x0] + [x0.clone() for _ in range(sets - 1)]
    per_row = op in ("cross_entropy", "row_sum", "row_minmax")
    ys2 = [torch.empty(rows, device=dev) for _ in range(sets)] if op == "row_minmax" else None
    if per_row:
        ys = [torch.empty(rows, device=dev) for _ in range(sets)]
    else:
        ys = [torch.empty_like(x0) for _ in range(sets)]
    g = torch.rand(cols, device=dev, generator=gen) + 0.5
    b = torch.randn(cols, device=dev, generator=gen) * 0.1
    if args.no_params:
        g = b = None
    lab = torch.randint(0, cols, (rows,), device=dev, generator=gen)
    rs = [torch.randn(rows, cols, device=dev, generator=gen) for _ in range(sets)] if op == "add_layernorm" else None
    ws = torch.empty(rows * 64 * 8, dtype=torch.uint8, device=dev)  # the largest split: 64 segments
    run = _launcher(op, xs, ys, g, b, lab, rows, cols, args.eps, args.policy, sh, rs, ys2, ws)

    facts = lr.lr_device_facts_query()
    aligned = 1 if cols % 4 == 0 else 0
    # without parameters a norm's typed call may take a plan of its own,
    # which the plan query does not report: time the call itself (plan None)
    auto = None if args.no_params else lr.lr_plan_query(op, rows, cols, args.policy)
    lr.check(run(0, auto), "automatic plan")
    torch.cuda.synchronize()
    ref = ys[0].double().clone()
    bound = 1e-6 + 1e-5 * ref.abs()

    timer = _time_graph if args.graph else _time
    if args.compare:
        return _compare(args, op, rows, cols, aligned, facts, auto, run, ys, ref, bound, timer, stream)
    results = []
    for p in lr.lr_plan_enumerate(facts, op, rows, cols, args.policy, aligned):
        # whole-wave plans: at most that many rows per workgroup; sub-wave
        # plans (several rows per wave): at most that many waves
        packed = p.threads_per_block // 64 if p.lanes_per_row < 64 else p.rows_per_block
        if packed > args.max_rows_per_block:
            continue
        st = run(0, p)
        torch.cuda.synchronize()
        valid = st == lr.LR_OK and bool(((ys[0].double() - ref).abs() <= bound).all())
        us = timer(run, p, args.iters, stream) if valid else float("inf")
        rec = dict(plan=p.as_dict(), us=us, valid=valid)
        results.append((us, p, rec))
        if args.json:
            print(json.dumps(rec), flush=True)
    results.sort(key=lambda t: t[0])
    best_us, best, _ = results[0]
    again = timer(run, best, args.iters, stream)
    moved = {"cross_entropy": tensor_bytes + rows * 12, "add_layernorm": 3 * tensor_bytes,
             "row_sum": tensor_bytes + rows * 4, "row_minmax": tensor_bytes + rows * 8}.get(op, 2 * tensor_bytes)
    print(f"# {op} {rows}x{cols} {args.policy}{' (graph)' if args.graph else ''}: {len(results)} candidates, "
          f"automatic {timer(run, auto, args.iters, stream):.2f} us, "
          f"best {again:.2f} us ({moved / again / 1e3:.0f} GB/s): {best!r}")
    for us, p, rec in results[:8]:
        print(f"#   {us:8.2f} us  {p!r}")
    fam = {0: "LR_FAMILY_CACHE", 1: "LR_FAMILY_STREAM", 2: "LR_FAMILY_ORDERED", 3: "LR_FAMILY_TREE",
           4: "LR_FAMILY_SPLIT"}
    opn = {0: "LR_OP_SOFTMAX", 1: "LR_OP_RMSNORM", 2: "LR_OP_LAYERNORM", 3: "LR_OP_CROSS_ENTROPY",
           4: "LR_OP_ADD_LAYERNORM", 5: "LR_OP_ROW_SUM", 6: "LR_OP_ROW_MINMAX"}[lr.OPS[op]]
    pol = {"unordered_tree": "LR_UNORDERED_TREE", "ordered_fold": "LR_ORDERED_FOLD", "fold_left": "LR_ORDERED_FOLD",
           "ordered_tree": "LR_ORDERED_TREE", "fold_right": "LR_FOLD_RIGHT"}[args.policy]

    def table_line(p):
        splits = p.splits if p.family == lr.LR_FAMILY_SPLIT else 0
        lanes = p.lanes_per_row if p.lanes_per_row < 64 else 0
        # trailing fields: splits, lanes per row, 1 for a no-parameter entry
        extra = [splits, lanes] + ([1] if args.no_params else [])
        while extra and extra[-1] == 0:
            extra.pop()
        tail = "".join(f", {v}" for v in extra)
        return (f"{{{opn}, {pol}, {rows}, {cols}, {aligned}, {fam[p.family]}, {p.waves_per_row}, "
                f"{p.rows_per_block}, {p.chunks_per_lane}{tail}}},")
    # the best plan, and the best that needs no workspace (the typed entry
    # points' choice) when the best splits rows
    print(table_line(best))
    if best.family == lr.LR_FAMILY_SPLIT:
        free = next(t for t in results if t[1].family != lr.LR_FAMILY_SPLIT)
        print(f"# best without a workspace: {free[0]:.2f} us")
        print(table_line(free[1]))
    return 0


if __name__ == "__main__":
    sys.exit(main())
