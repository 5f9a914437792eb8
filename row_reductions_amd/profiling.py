"""HBM traffic from rocprofv3 counter runs, tied to the kernel sources.

Two `rocprofv3 --pmc` runs of the benchmark (one with FETCH_SIZE, one with
WRITE_SIZE, both launched with `bench.py --copy-probe`) give KiB per
dispatch for every kernel.  The counters are calibrated against a plain
device-to-device copy of known size that runs in the same process (the last
20 `__amd_rocclr_copyBuffer` dispatches): bytes = counter * (known bytes /
copy's counter).  The summary records a hash of the device sources (the
`.hip` translation units and the headers they compile), so a figure taken
before a kernel change is not reported for the changed kernel; a lookup also
names the exact kernel instance the caller's plan launches.

    python -m row_reductions_amd.profiling traffic --fetch F.csv --write W.csv \\
        --copy-bytes 18874368 --out profiles/hbm_traffic_768x6144.json
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
OP_NAMES = {0: "softmax", 1: "rmsnorm", 2: "layernorm", 3: "cross_entropy"}


def csrc_hash() -> str:
    """sha256 over the device sources: the `.hip` translation units and the
    `.hpp` headers (names and contents), and the compiler flags they are
    built with (include paths left out: they name the checkout).  Host-only
    files (the C ABI, the planner and its table) do not change a kernel."""
    from . import build as _build
    h = hashlib.sha256()
    flags = [f for f in _build.COMMON if not f.startswith("-I")]
    h.update(repr((flags, sorted(_build.EXTRA.items()))).encode())
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def _per_kernel(path: str):
    vals = defaultdict(list)
    order = []
    with open(path) as f:
        for r in csv.DictReader(f):
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
            order.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return vals, order


def counter_means(path: str) -> dict:
    """Per kernel, the mean over its dispatches of every counter in a
    rocprofv3 counter-collection CSV (one row per dispatch and counter)."""
    acc = defaultdict(lambda: defaultdict(list))
    with open(path) as f:
        for r in csv.DictReader(f):
            acc[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = {}
    for name, per in acc.items():
        rec = {c: sum(v) / len(v) for c, v in per.items()}
        rec["dispatches"] = max(len(v) for v in per.values())
        out[name] = rec
    return out


def kernel_op(name: str):
    m = re.search(r"lr::k_(cache|stream|ordered)<(\d+)", name)
    return OP_NAMES.get(int(m.group(2))) if m else None


def traffic(fetch_csv: str, write_csv: str, copy_bytes: int) -> dict:
    out = {"csrc_sha256": csrc_hash(), "copy_bytes": copy_bytes, "kernels": {}}
    scale = {}
    per = {}
    for key, path in (("fetch", fetch_csv), ("write", write_csv)):
        vals, order = _per_kernel(path)
        probe = [v for n, v in order if "copyBuffer" in n][-20:]
        if not probe:
            raise SystemExit(f"{path}: no copy probe dispatches")
        copy_kib = sum(probe) / len(probe)
        scale[key] = copy_bytes / (copy_kib * 1024.0)
        out[f"copy_{key}_kib"] = copy_kib
        out[f"{key}_scale"] = scale[key]
        per[key] = vals
    for name in per["fetch"]:
        op = kernel_op(name)
        if op is None or name not in per["write"]:
            continue
        f_kib = sum(per["fetch"][name]) / len(per["fetch"][name])
        w_kib = sum(per["write"][name]) / len(per["write"][name])
        out["kernels"][name] = {
            "op": op,
            "fetch_kib": f_kib,
            "write_kib": w_kib,
            "fetch_bytes": f_kib * 1024.0 * scale["fetch"],
            "write_bytes": w_kib * 1024.0 * scale["write"],
            "traffic_bytes": f_kib * 1024.0 * scale["fetch"] + w_kib * 1024.0 * scale["write"],
            "dispatches": len(per["fetch"][name]),
        }
    return out


def trace(trace_csv: str, kernels: list[str] | None = None) -> dict:
    """Per-kernel dispatch count and average / median / minimum / maximum
    duration in microseconds from a `rocprofv3 --kernel-trace` CSV, for the
    row-reduction kernels (or the named ones)."""
    durs = defaultdict(list)
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if (kernels and name not in kernels) or (not kernels and kernel_op(name) is None):
                continue
            durs[name].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = {"csrc_sha256": csrc_hash(), "kernels": {}}
    for name, d in durs.items():
        d.sort()
        out["kernels"][name] = {"op": kernel_op(name), "dispatches": len(d), "avg_us": sum(d) / len(d),
                                "median_us": d[len(d) // 2], "min_us": d[0], "max_us": d[-1]}
    return out


def trace_runs(trace_csv: str, min_dispatches: int = 100) -> list[dict]:
    """Consecutive runs of dispatches of one kernel instance with one grid
    size, in trace order, with their count and average / median duration
    (us): the phases of a script that times one shape after another.  Runs
    shorter than `min_dispatches` (calibration, warm-up calls) are left out."""
    import gzip
    opener = gzip.open if trace_csv.endswith(".gz") else open
    rows = []
    with opener(trace_csv, "rt") as f:
        for r in csv.DictReader(f):
            grid = r.get("Grid_Size_X") or r.get("Grid_Size")
            rows.append((int(r["Start_Timestamp"]), r["Kernel_Name"], int(grid),
                         (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    rows.sort()
    runs, cur = [], None
    for _, name, grid, d in rows:
        if cur is None or (name, grid) != (cur["kernel"], cur["grid"]):
            cur = {"kernel": name, "grid": grid, "durs": []}
            runs.append(cur)
        cur["durs"].append(d)
    out = []
    for r in runs:
        d = sorted(r.pop("durs"))
        if len(d) >= min_dispatches:
            out.append(dict(r, dispatches=len(d), avg_us=sum(d) / len(d), median_us=d[len(d) // 2]))
    return out


# Parameter list of every kernel entry (csrc/lr_entry.hpp), as demangled:
# the nine preloaded leading arguments, then KArgs.
ENTRY_PARAMS = ("(float const*, long, int, int, int, int, float const*, float const*, float const*, "
                "lr::KArgs)")


def kernel_name(op_index: int, plan, aligned: bool, param_mode: int) -> str | None:
    """The demangled name of the kernel instance a CACHE or STREAM plan
    launches (param_mode: 0 no gamma/beta, 1 all present, 2 some)."""
    al = "true" if aligned else "false"
    if plan.family == 0:
        return f"void lr::k_cache<{op_index}, {plan.chunks_per_lane}, {al}, {param_mode}>" + ENTRY_PARAMS
    if plan.family == 1:
        return f"void lr::k_stream<{op_index}, {al}>" + ENTRY_PARAMS
    return None


def lookup(summary_path: str, op: str, kernel: str | None = None):
    """Traffic record of `op` if the summary matches the current device
    sources and, when `kernel` is given, was taken for that kernel."""
    try:
        with open(summary_path) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    if s.get("csrc_sha256") != csrc_hash():
        return None
    for name, rec in s.get("kernels", {}).items():
        if rec.get("op") == op and (kernel is None or name == kernel):
            return dict(rec, kernel=name)
    return None


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--command", default="", help="the profiling command, recorded in the summary")
    t.add_argument("--out", required=True)
    tr = sub.add_parser("trace")
    tr.add_argument("--trace", required=True, help="rocprofv3 kernel-trace CSV")
    tr.add_argument("--command", default="", help="the profiling command, recorded in the summary")
    tr.add_argument("--out", required=True)
    ru = sub.add_parser("runs")
    ru.add_argument("--trace", required=True, help="rocprofv3 kernel-trace CSV (or .csv.gz)")
    ru.add_argument("--min-dispatches", type=int, default=100)
    sub.add_parser("hash")
    co = sub.add_parser("counters")
    co.add_argument("--csv", required=True, help="rocprofv3 counter-collection CSV")
    a = ap.parse_args(argv)
    if a.cmd == "counters":
        for name, rec in counter_means(a.csv).items():
            vals = "  ".join(f"{c} {v:.6g}" for c, v in sorted(rec.items()) if c != "dispatches")
            print(f"{rec['dispatches']:6d} dispatches  {vals}  {name}")
        return 0
    if a.cmd == "runs":
        for r in trace_runs(a.trace, a.min_dispatches):
            print(f"{r['dispatches']:7d} dispatches  grid {r['grid']:9d}  avg {r['avg_us']:8.3f} us  "
                  f"median {r['median_us']:8.3f} us  {r['kernel']}")
        return 0
    if a.cmd == "hash":
        print(csrc_hash())
        return 0
    if a.cmd == "trace":
        s = trace(a.trace)
        s["command"] = a.command
        with open(a.out, "w") as f:
            json.dump(s, f, indent=1)
        for name, rec in s["kernels"].items():
            print(f"{rec['op']:14s} {rec['dispatches']:7d} dispatches  avg {rec['avg_us']:8.3f} us  "
                  f"median {rec['median_us']:8.3f} us  {name}")
        return 0
    s = traffic(a.fetch, a.write, a.copy_bytes)
    s["command"] = a.command
    with open(a.out, "w") as f:
        json.dump(s, f, indent=1)
    for name, rec in s["kernels"].items():
        print(f"{rec['op']:14s} fetch {rec['fetch_bytes'] / 1e6:8.2f} MB  write {rec['write_bytes'] / 1e6:8.2f} MB  "
              f"{name}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
