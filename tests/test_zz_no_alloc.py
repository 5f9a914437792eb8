"""lr_run_f32_noalloc (the entry point for callers that cannot allocate device
memory) against lr_run_f32 with a caller workspace: the same plan gives the
same bits, on consecutive calls whose second is smaller, through the C ABI.
Each output is also held to the oracle's bar."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import row_reductions_amd as lr
import synth
from gpu_util import ATOL, DEV, RTOL

pytestmark = pytest.mark.gpu


def _split_plan(op, rows, cols, splits, aligned):
    for p in lr.lr_plan_enumerate(lr.lr_device_facts_query(), op, rows, cols, "unordered_tree", aligned):
        if p.family == lr.LR_FAMILY_SPLIT and p.splits == splits:
            return p
    raise AssertionError(f"no split plan with {splits} segments for {op} {rows}x{cols}")


def _inputs(op, rows, cols, seed):
    if op == "add_layernorm":
        return synth.add_layernorm_inputs(rows, cols, seed=seed, mean=3.0, std=2.0)
    if op == "layernorm":
        return synth.layernorm_inputs(rows, cols, seed=seed, mean=3.0, std=2.0)
    if op == "cross_entropy":
        return synth.cross_entropy_inputs(rows, cols, seed=seed)
    return synth.softmax_inputs(rows, cols, seed=seed, std=4.0)


def _run_both(op, inp, rows, cols, plan):
    """(output of lr_run_f32 with a workspace, output of lr_run_f32_noalloc)."""
    d = {k: torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for k, v in inp.items()}
    outs = []
    for noalloc in (False, True):
        if op == "cross_entropy":
            out = torch.full((rows,), float("nan"), device=DEV)
            t = dict(x=d["logits"], labels=d["labels"], losses=out)
        else:
            out = torch.full((rows, cols), float("nan"), device=DEV)
            t = dict(x=d["x"], y=out)
            if op == "add_layernorm":
                t.update(residual=d["residual"], gamma=d["gamma"], beta=d["beta"])
            elif op == "layernorm":
                t.update(gamma=d["gamma"], beta=d["beta"])
        eps = 1e-5 if op in ("layernorm", "add_layernorm") else 0.0
        if noalloc:
            st = lr.lr_run_f32_noalloc(op, rows, cols, eps, "unordered_tree", plan, **t)
        else:
            n = max(lr.lr_workspace_query(op, rows, cols), lr.lr_plan_workspace_bytes(plan, rows), 16)
            ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=DEV)
            st = lr.lr_run_f32(op, rows, cols, eps, "unordered_tree", plan, ws, **t)
        assert st == lr.LR_OK, (op, noalloc, lr.lr_status_string(st))
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    return outs


def _ref(op, inp):
    if op == "add_layernorm":
        return oracle.add_layernorm(inp["x"], inp["residual"], inp["gamma"], inp["beta"], 1e-5)
    if op == "layernorm":
        return oracle.layernorm(inp["x"], inp["gamma"], inp["beta"], 1e-5)
    if op == "cross_entropy":
        return oracle.cross_entropy(inp["logits"], inp["labels"])
    return oracle.softmax(inp["x"])


# each pair: a call, then a smaller one; None is the automatic plan (which
# splits the fused residual LayerNorm at 64 x 12288 by itself)
PAIRS = [
    ("layernorm", (64, 12289, 4), (16, 3001, 8)),
    ("add_layernorm", (64, 12288, None), (8, 4096, None)),
    ("softmax", (32, 20000, 16), (5, 999, 2)),
    ("cross_entropy", (48, 32000, 8), (7, 4096, 4)),
]


@pytest.mark.parametrize("op,first,second", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_matches_the_workspace_entry_point(op, first, second):
    for k, (rows, cols, splits) in enumerate((first, second)):
        print(f"\n[gpu] noalloc {op} {rows}x{cols} splits={splits}", flush=True)
        plan = None if splits is None else _split_plan(op, rows, cols, splits, 1 if cols % 4 == 0 else 0)
        inp = _inputs(op, rows, cols, seed=rows + k)
        a, b = _run_both(op, inp, rows, cols, plan)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (op, rows, cols)
        ref = _ref(op, inp)
        err = np.abs(b.astype(np.float64) - ref)
        assert (err <= ATOL + RTOL * np.abs(ref)).all(), (op, rows, cols, float(err.max()))


def test_noalloc_refuses_a_plan_larger_than_its_array():
    rows, cols = 4096, 1024
    plan = _split_plan("softmax", rows, cols, 64, 1)
    assert lr.lr_plan_workspace_bytes(plan, rows) > (1 << 20)
    x = torch.randn(rows, cols, device=DEV)
    y = torch.full_like(x, 7.0)
    st = lr.lr_run_f32_noalloc("softmax", rows, cols, 0.0, "unordered_tree", plan, x=x, y=y)
    assert st == lr.LR_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())  # nothing launched
    # the same array then serves a plan that fits
    small = _split_plan("softmax", 64, cols, 8, 1)
    xs, ys = x[:64].contiguous(), torch.empty(64, cols, device=DEV)
    assert lr.lr_run_f32_noalloc("softmax", 64, cols, 0.0, "unordered_tree", small, x=xs, y=ys) == lr.LR_OK
    torch.cuda.synchronize()
    ref = oracle.softmax(xs.cpu().numpy())
    assert (np.abs(ys.cpu().numpy() - ref) <= ATOL + RTOL * np.abs(ref)).all()
