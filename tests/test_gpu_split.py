"""Split-row family on the GPU, through lr_run_f32 and a caller workspace:
rows too few to fill the device are cut into segments whose partial
statistics merge in a second kernel (max / rescaled sum of exp; mean and
M2 by the pairwise update of Chan, Golub and LeVeque for LayerNorm).
Parity against the double oracle at the LayerNorm workload shape (64 x
12289) for every operation, every split plan on ragged shapes (including
segments with no chunk), misaligned bases, in place, workspace canaries,
the unsplit fallback for a short workspace, and HIP graph replay."""
import numpy as np
import pytest
import torch

import oracle
import row_reductions_amd as lr
import synth
from gpu_util import DEV, assert_parity, check_output, run_gpu, workspace_for

pytestmark = pytest.mark.gpu

OPS = ["softmax", "rmsnorm", "layernorm", "cross_entropy", "add_layernorm", "row_sum", "row_minmax"]
EPS = {"rmsnorm": 1e-6, "layernorm": 1e-5, "add_layernorm": 1e-5}
GEN = {"softmax": dict(std=4.0), "rmsnorm": {}, "layernorm": dict(mean=3.0, std=2.0), "cross_entropy": {},
       "add_layernorm": dict(mean=3.0, std=2.0)}


def inputs(op, rows, cols, seed):
    if op in GEN:
        return synth.make_inputs(op, rows, cols, seed=seed, **GEN[op])
    return {"x": synth.normal_f32(seed, 0, rows * cols, 0.25, 3.0).reshape(rows, cols)}


def place(a, pad=0, canary=None):
    """`a` (or an empty rows x cols buffer) `pad` floats into a larger buffer."""
    rows, cols = a.shape
    full = torch.full((rows * cols + 2 * pad + 8,), canary if canary is not None else float("nan"), device=DEV)
    v = full[pad:pad + rows * cols].view(rows, cols)
    v.copy_(torch.from_numpy(np.ascontiguousarray(a)).to(DEV))
    return v, full


def run(op, inp, plan=None, workspace=None, workspace_bytes=None, pad=0, in_place=False):
    """One lr_run_f32 call; returns (status, dict of numpy outputs)."""
    x = inp["logits"] if op == "cross_entropy" else inp["x"]
    rows, cols = x.shape
    xv, _ = place(x, pad)
    t = {"x": xv}
    out = {}
    if op in ("softmax", "rmsnorm", "layernorm", "add_layernorm"):
        t["y"] = xv if in_place else place(np.zeros_like(x), pad)[0]
        out["y"] = t["y"]
        if op != "softmax" and inp.get("gamma") is not None:
            t["gamma"] = torch.from_numpy(inp["gamma"]).to(DEV)
        if op in ("layernorm", "add_layernorm") and inp.get("beta") is not None:
            t["beta"] = torch.from_numpy(inp["beta"]).to(DEV)
        if op == "add_layernorm":
            t["residual"] = place(inp["residual"], pad)[0]
            t["sum_out"] = place(np.zeros_like(x), pad)[0]
            out["sum_out"] = t["sum_out"]
    elif op == "cross_entropy":
        t["labels"] = torch.from_numpy(inp["labels"]).to(DEV)
        t["losses"] = out["y"] = torch.full((rows,), float("nan"), device=DEV)
    elif op == "row_sum":
        t["sums"] = out["y"] = torch.full((rows,), float("nan"), device=DEV)
    else:
        t["mins"] = out["mins"] = torch.full((rows,), float("nan"), device=DEV)
        t["maxs"] = out["maxs"] = torch.full((rows,), float("nan"), device=DEV)
    st = lr.lr_run_f32(op, rows, cols, EPS.get(op, 0.0), "unordered_tree", plan, workspace, workspace_bytes,
                       None, **t)
    torch.cuda.synchronize()
    return st, {k: v.cpu().numpy() for k, v in out.items()}


def check(op, inp, got, what):
    x = inp["logits"] if op == "cross_entropy" else inp["x"]
    if op == "add_layernorm":
        ref, ref_s = oracle.add_layernorm(x, inp["residual"], inp.get("gamma"), inp.get("beta"), EPS[op],
                                          with_sum=True)
        assert np.array_equal(got["sum_out"].view(np.uint32), ref_s.view(np.uint32)), f"{what}: combined input"
        assert_parity(got["y"], ref, what)
    elif op == "row_sum":
        ref = oracle.row_sum(x)
        bound = 1e-6 + 1e-5 * np.abs(x.astype(np.float64)).sum(axis=1)
        assert (np.abs(got["y"].astype(np.float64) - ref) <= bound).all(), what
    elif op == "row_minmax":
        lo, hi = oracle.row_minmax(x)
        assert np.array_equal(got["mins"], lo) and np.array_equal(got["maxs"], hi), what
    else:
        check_output(op, inp, EPS.get(op), "unordered_tree", got["y"], what)


def split_plan(op, rows, cols, G=4, S=4):
    facts = lr.lr_device_facts_query()
    return next(p for p in lr.lr_plan_enumerate(facts, op, rows, cols, "unordered_tree", 1 if cols % 4 == 0 else 0)
                if p.family == lr.LR_FAMILY_SPLIT and p.splits == G and p.waves_per_row == S)


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("cols", [12289, 12288])
def test_split_at_the_layernorm_workload_shape(op, cols):
    """the fused residual LayerNorm splits automatically at 64 x 12288; every
    op splits under an explicit plan, and a fixed plan gives the same bits
    twice"""
    rows = 64
    print(f"\n[gpu] split {op} {rows}x{cols}", flush=True)
    need = lr.lr_workspace_query(op, rows, cols)
    facts = lr.lr_device_facts_query()
    auto = lr.lr_plan_for_device_ws(facts, op, rows, cols, "unordered_tree", 1 if cols % 4 == 0 else 0)
    auto_splits = op == "add_layernorm" and cols == 12288
    plan = auto if auto_splits else split_plan(op, rows, cols)
    assert plan.family == lr.LR_FAMILY_SPLIT
    if not auto_splits:
        assert need == 0 and auto.family != lr.LR_FAMILY_SPLIT  # one launch is faster
    ws = torch.full((lr.lr_plan_workspace_bytes(plan, rows),), 0xFF, dtype=torch.uint8, device=DEV)
    inp = inputs(op, rows, cols, seed=cols + len(op))
    st, got = run(op, inp, plan=plan, workspace=ws)
    assert st == lr.LR_OK, lr.lr_status_string(st)
    check(op, inp, got, f"{op} {rows}x{cols} split")
    st2, got2 = run(op, inp, plan=plan, workspace=ws)
    assert st2 == lr.LR_OK
    for k in got:
        assert np.array_equal(got[k].view(np.uint32), got2[k].view(np.uint32)), k
    if auto_splits:  # the automatic plan with the queried workspace
        assert need >= lr.lr_plan_workspace_bytes(plan, rows) > 0
        st3, got3 = run(op, inp, workspace=torch.empty(need, dtype=torch.uint8, device=DEV))
        assert st3 == lr.LR_OK
        for k in got:
            assert np.array_equal(got[k].view(np.uint32), got3[k].view(np.uint32)), k


SHAPES = [(3, 20), (2, 21), (5, 257), (4, 1537), (2, 6144), (3, 12289)]


@pytest.mark.parametrize("op", OPS)
def test_every_split_plan(op):
    facts = lr.lr_device_facts_query()
    n = 0
    for rows, cols in SHAPES:
        inp = inputs(op, rows, cols, seed=rows * 7 + cols)
        plans = [p for p in lr.lr_plan_enumerate(facts, op, rows, cols, "unordered_tree", 1 if cols % 4 == 0 else 0)
                 if p.family == lr.LR_FAMILY_SPLIT]
        assert plans, (rows, cols)
        print(f"\n[gpu] split plans {op} {rows}x{cols}: {len(plans)}", flush=True)
        for p in plans:
            st, got = run(op, inp, plan=p, workspace=workspace_for(p, rows))
            assert st == lr.LR_OK, (p, lr.lr_status_string(st))
            check(op, inp, got, f"{op} {rows}x{cols} {p}")
            n += 1
    assert n > 100


@pytest.mark.parametrize("op", OPS)
def test_split_misaligned_bases(op):
    facts = lr.lr_device_facts_query()
    for pad in (1, 2, 3):
        for rows, cols in [(4, 4096), (3, 12289)]:
            inp = inputs(op, rows, cols, seed=pad + cols)
            p = next(q for q in lr.lr_plan_enumerate(facts, op, rows, cols, "unordered_tree", 0)
                     if q.family == lr.LR_FAMILY_SPLIT and q.splits == 8)
            st, got = run(op, inp, plan=p, workspace=workspace_for(p, rows), pad=pad)
            assert st == lr.LR_OK
            check(op, inp, got, f"{op} pad {pad} {rows}x{cols}")


@pytest.mark.parametrize("op", ["softmax", "rmsnorm", "layernorm", "add_layernorm"])
def test_split_in_place(op):
    rows, cols = 64, 12289
    inp = inputs(op, rows, cols, seed=5)
    p = split_plan(op, rows, cols)
    st, got = run(op, inp, plan=p, workspace=workspace_for(p, rows), in_place=True)
    assert st == lr.LR_OK
    check(op, inp, got, f"{op} in place")


def test_split_layernorm_large_mean_small_spread():
    """mean 1000, std 1e-2.  No FP32 LayerNorm meets the parity bar here (an
    FP32 row sum near 1.2e7 carries a mean error near 1e-4, 1% of the
    spread), so the split result is held to the workspace-free kernel's own
    error against the double oracle: the merged M2 adds no cancellation (an
    E[x^2] - E[x]^2 merge would lose the variance entirely at this scale),
    and the output keeps the variance var / (var + eps)."""
    rows, cols = 64, 12289
    x = synth.normal_f32(9, 0, rows * cols, 1000.0, 1e-2).reshape(rows, cols)
    inp = {"x": x, "gamma": None, "beta": None}
    ref = oracle.layernorm(x, None, None, 1e-5)
    p = split_plan("layernorm", rows, cols)
    st, split = run("layernorm", inp, plan=p, workspace=workspace_for(p, rows))
    assert st == lr.LR_OK
    st, whole = run("layernorm", inp)
    assert st == lr.LR_OK
    e_split = np.abs(split["y"] - ref).max()
    e_whole = np.abs(whole["y"] - ref).max()
    print(f"\n[gpu] mean 1000: max |err| split {e_split:.3g}, unsplit {e_whole:.3g}", flush=True)
    assert e_split <= 2.0 * e_whole + 1e-5
    # the FP32 mean error shifts a row's outputs alike (as much as unsplit);
    # the spread is that of the normalised row
    ys, yw = split["y"].astype(np.float64), whole["y"].astype(np.float64)
    assert np.abs(ys.mean(axis=1)).max() <= 2.0 * np.abs(yw.mean(axis=1)).max() + 1e-4
    _, var = oracle.layernorm_stats(x)  # eps is not negligible beside var = 1e-4
    assert np.abs(ys.var(axis=1) - var / (var + np.float32(1e-5))).max() < 1e-3


def test_workspace_beyond_the_plan_is_untouched_and_short_workspace_runs_unsplit():
    rows, cols = 64, 12288
    op = "add_layernorm"
    inp = inputs(op, rows, cols, seed=8)
    facts = lr.lr_device_facts_query()
    plan = lr.lr_plan_for_device_ws(facts, op, rows, cols, "unordered_tree", 1)
    assert plan.family == lr.LR_FAMILY_SPLIT
    need = lr.lr_plan_workspace_bytes(plan, rows)
    big = torch.full((need + 4096,), 0x5A, dtype=torch.uint8, device=DEV)
    st, got = run(op, inp, plan=plan, workspace=big)
    assert st == lr.LR_OK
    check(op, inp, got, "big workspace")
    assert (big[need:].cpu().numpy() == 0x5A).all()
    # too small for the automatic split: the call runs the unsplit plan
    small = torch.full((need - 16,), 0x5A, dtype=torch.uint8, device=DEV)
    st, got2 = run(op, inp, workspace=small)
    assert st == lr.LR_OK
    check(op, inp, got2, "short workspace")
    assert (small.cpu().numpy() == 0x5A).all()
    # an explicit split plan with that workspace is an error, not a fallback
    st, _ = run(op, inp, plan=plan, workspace=small)
    assert st == lr.LR_ERR_WORKSPACE


def test_split_cross_entropy_labels_out_of_range():
    rows, cols = 64, 12289
    inp = inputs("cross_entropy", rows, cols, seed=4)
    inp["labels"][::5] = -1
    inp["labels"][1::7] = cols
    inp["labels"][2::11] = np.int64(1) << 40
    p = split_plan("cross_entropy", rows, cols)
    st, got = run("cross_entropy", inp, plan=p, workspace=workspace_for(p, rows))
    assert st == lr.LR_OK
    check("cross_entropy", inp, got, "labels out of range")


def test_split_under_graph_replay():
    rows, cols = 64, 12289
    inp = inputs("layernorm", rows, cols, seed=2)
    x = torch.from_numpy(inp["x"]).to(DEV)
    g, b = torch.from_numpy(inp["gamma"]).to(DEV), torch.from_numpy(inp["beta"]).to(DEV)
    p = split_plan("layernorm", rows, cols)
    ws = workspace_for(p, rows)
    eager = torch.empty_like(x)
    lr.check(lr.lr_layernorm_f32(x, g, b, eager, rows, cols, 1e-5, plan=p, workspace=ws))
    torch.cuda.synchronize()
    out = torch.full_like(x, float("nan"))
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            lr.check(lr.lr_layernorm_f32(x, g, b, out, rows, cols, 1e-5, stream=torch.cuda.current_stream(),
                                         plan=p, workspace=ws))
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        ws.fill_(0xFF)  # the partials must come from this replay
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32)), rep
        lr.check(lr.lr_layernorm_f32(x, g, b, eager, rows, cols, 1e-5, plan=p, workspace=ws))
        torch.cuda.synchronize()
