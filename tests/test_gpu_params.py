"""gamma and beta at every 4-byte offset from the 16-byte grid, against rows
at every phase, on the GPU: one plan of each family that reads the
parameters (whole-wave and sub-wave CACHE, STREAM, split rows through a
workspace), each within |gpu - ref| <= 1e-6 + 1e-5 |ref| of the double
oracle ("TIRx Metal reduction lowering", section 8, the affine step).
Parameters off the grid make every call take the misaligned kernels, which
read a parameter chunk as one 16-byte read at a 4-byte aligned offset, or
(a row's first and last chunk, and rows packed several to a wave) as the two
16-byte blocks of the parameter's own grid that cover it."""
import numpy as np
import pytest
import torch

import oracle
import row_reductions_amd as lr
import synth
from gpu_util import DEV, assert_parity, guards_intact, placed

pytestmark = pytest.mark.gpu

OPS = ["rmsnorm", "layernorm", "add_layernorm"]
EPS = {"rmsnorm": 1e-6, "layernorm": 1e-5, "add_layernorm": 1e-5}
SHAPES = [(157, 50), (157, 64), (40, 1537), (8, 6147)]  # narrow rows, then whole waves
OFFSETS = [(0, 1, 2), (1, 3, 0), (2, 2, 2), (3, 0, 1)]  # (x and y, gamma, beta) in floats


def plans_for(op, rows, cols):
    """the first legal plan of each family for unaligned calls, plus a
    sub-wave CACHE plan where there is one, and for whole-wave teams one with
    several chunks per lane at one and at several waves per row (there only a
    row's first and last chunk take the two-block read, in the waves that
    hold them)"""
    facts = lr.lr_device_facts_query()
    out = {}
    for p in lr.lr_plan_enumerate(facts, op, rows, cols, "unordered_tree", 0):
        key = (p.family, p.lanes_per_row < 64 * p.waves_per_row, min(p.chunks_per_lane, 2), min(p.waves_per_row, 2))
        out.setdefault(key, p)
    return list(out.values())


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("op", OPS)
def test_parameters_off_the_grid(op, rows, cols):
    if op == "rmsnorm":
        d = synth.rmsnorm_inputs(rows, cols, seed=11)
    elif op == "layernorm":
        d = synth.layernorm_inputs(rows, cols, seed=12, mean=3.0, std=2.0)
    else:
        d = synth.add_layernorm_inputs(rows, cols, seed=13, mean=3.0, std=2.0)
    x, gam = d["x"], d["gamma"]
    bet = d.get("beta")
    if op == "rmsnorm":
        ref = oracle.rmsnorm(x, gam, EPS[op])
    elif op == "layernorm":
        ref = oracle.layernorm(x, gam, bet, EPS[op])
    else:
        ref = oracle.add_layernorm(x, d["residual"], gam, bet, EPS[op])
    plans = plans_for(op, rows, cols)
    assert {p.family for p in plans} >= {lr.LR_FAMILY_CACHE, lr.LR_FAMILY_STREAM}
    for xo, go, bo in OFFSETS:
        for plan in [None] + plans:
            what = f"{op} {rows}x{cols} x/y+{xo} gamma+{go} beta+{bo} plan={plan}"
            print(f"\n[gpu] params {what}", flush=True)
            xv, _ = placed(x, xo)
            yv, yf = placed(np.zeros_like(x), xo)
            gv, _ = placed(gam, go)
            bv = placed(bet, bo)[0] if bet is not None else None
            ws = None
            if plan is not None and plan.family == lr.LR_FAMILY_SPLIT:
                ws = torch.zeros(lr.lr_plan_workspace_bytes(plan, rows), dtype=torch.uint8, device=DEV)
            if op == "rmsnorm":
                st = lr.lr_rmsnorm_f32(xv, gv, yv, rows, cols, EPS[op], plan=plan, workspace=ws)
            elif op == "layernorm":
                st = lr.lr_layernorm_f32(xv, gv, bv, yv, rows, cols, EPS[op], plan=plan, workspace=ws)
            else:
                rv, _ = placed(d["residual"], xo)
                st = lr.lr_add_layernorm_f32(xv, rv, gv, bv, yv, None, rows, cols, EPS[op], plan=plan,
                                             workspace=ws)
            torch.cuda.synchronize()
            assert st == lr.LR_OK, (what, lr.lr_status_string(st))
            assert guards_intact(yv, yf), what
            assert_parity(yv.cpu().numpy(), ref, what)


def test_rmsnorm_without_gamma_takes_its_own_plan():
    """RMSNorm 768x6144 called without gamma launches the plan listed for that
    case (five waves of six chunks per row), not the four waves of six of the
    call with gamma: its output equals that explicit plan's bit for bit (the
    unordered tree is fixed by the plan) and the double oracle within the
    stated bound ("TIRx Metal reduction lowering", section 8, the affine step
    skipped when no scale is given)"""
    rows, cols = 768, 6144
    d = synth.rmsnorm_inputs(rows, cols, seed=21)
    x = d["x"]
    ref = oracle.rmsnorm(x, None, EPS["rmsnorm"])
    facts = lr.lr_device_facts_query()
    with_gamma = lr.lr_plan_query("rmsnorm", rows, cols, "unordered_tree")
    own = next(p for p in lr.lr_plan_enumerate(facts, "rmsnorm", rows, cols, "unordered_tree", 1)
               if p.family == lr.LR_FAMILY_CACHE and p.waves_per_row == 5 and p.chunks_per_lane == 6
               and p.rows_per_block == 1)
    assert (with_gamma.waves_per_row, with_gamma.chunks_per_lane) != (5, 6)
    xv = torch.from_numpy(x).to(DEV)
    outs = {}
    for name, plan in (("auto", None), ("own", own), ("with_gamma_plan", with_gamma)):
        print(f"\n[gpu] rmsnorm {rows}x{cols} without gamma plan={name}", flush=True)
        y = torch.zeros_like(xv)
        st = lr.lr_rmsnorm_f32(xv, None, y, rows, cols, EPS["rmsnorm"], plan=plan)
        torch.cuda.synchronize()
        assert st == lr.LR_OK, (name, lr.lr_status_string(st))
        outs[name] = y.cpu().numpy()
        assert_parity(outs[name], ref, f"rmsnorm without gamma, plan {name}")
    assert np.array_equal(outs["auto"].view(np.uint32), outs["own"].view(np.uint32))
