"""GPU parity of the fused residual LayerNorm through the C ABI.

combined = fl32(x + residual) and y = LayerNorm(combined) ("TIRx Metal
reduction lowering", section 5.1).  unordered_tree outputs meet
|gpu - ref| <= 1e-6 + 1e-5 |ref| against the double oracle; ordered_fold
outputs equal the CPU FP32 left-fold replay of LayerNorm over the oracle's
FP32 combined tensor bit for bit; the optional combined output equals the
oracle's FP32 sum bit for bit under every policy and plan."""
import numpy as np
import pytest
import torch

import oracle
import row_reductions_amd as lr
import synth
from gpu_util import DEV, assert_parity, dev, workspace_for

pytestmark = pytest.mark.gpu

EPS = 1e-5


def run_add(inp, policy="unordered_tree", plan=None, with_sum=True, affine=True, mode="plain", pads=(0, 0, 0, 0)):
    """mode: plain | y_is_x | y_is_res | sum_is_x | sum_is_res.  pads: float
    offsets of x, residual, y, sum inside larger buffers (misaligned bases)."""
    x, r = inp["x"], inp["residual"]
    rows, cols = x.shape
    n = rows * cols

    def place(a, pad):
        full = torch.empty(n + pad + 8, dtype=torch.float32, device=DEV)
        v = full[pad:pad + n].view(rows, cols)
        if a is not None:
            v.copy_(torch.from_numpy(a).to(DEV))
        return v

    xv, rv = place(x, pads[0]), place(r, pads[1])
    yv = {"y_is_x": xv, "y_is_res": rv}.get(mode)
    if yv is None:
        yv = place(None, pads[2])
    sv = None
    if with_sum:
        sv = {"sum_is_x": xv, "sum_is_res": rv}.get(mode)
        if sv is None:
            sv = place(None, pads[3])
    g = dev(inp["gamma"]) if affine else None
    b = dev(inp["beta"]) if affine else None
    st = lr.lr_add_layernorm_f32(xv, rv, g, b, yv, sv, rows, cols, EPS, policy, plan=plan,
                                 workspace=workspace_for(plan, rows))
    torch.cuda.synchronize()
    return st, yv.cpu().numpy(), (sv.cpu().numpy() if sv is not None else None)


def check(inp, policy, got_y, got_s, affine=True, what=""):
    g = inp["gamma"] if affine else None
    b = inp["beta"] if affine else None
    ref, ref_s = oracle.add_layernorm(inp["x"], inp["residual"], g, b, EPS, with_sum=True)
    if got_s is not None:
        assert np.array_equal(got_s.view(np.uint32), ref_s.view(np.uint32)), f"{what}: combined output"
    if policy == "ordered_fold":
        rep = oracle.layernorm_fold_f32(ref_s, g, b, EPS)
        if not np.array_equal(got_y.view(np.uint32), rep.view(np.uint32)):
            bad = tuple(np.argwhere(got_y.view(np.uint32) != rep.view(np.uint32))[0])
            raise AssertionError(f"{what}: differs from the FP32 replay at {bad}: {got_y[bad]!r} vs {rep[bad]!r}")
        return 0.0
    return assert_parity(got_y, ref, what)


def test_add_layernorm_768x6144_both_policies():
    inp = synth.add_layernorm_inputs(768, 6144, seed=0)
    for policy in ("unordered_tree", "ordered_fold"):
        print(f"\n[gpu] add_layernorm 768x6144 {policy}", flush=True)
        st, y, s = run_add(inp, policy)
        assert st == lr.LR_OK, lr.lr_status_string(st)
        worst = check(inp, policy, y, s, what=f"768x6144 {policy}")
        print(f"[gpu] add_layernorm 768x6144 {policy}: worst err/bound {worst:.3g}", flush=True)


COLS = [1, 3, 4, 5, 63, 64, 65, 255, 256, 1023, 1537, 4096, 6144, 12289, 40000]


@pytest.mark.parametrize("policy", ["unordered_tree", "ordered_fold"])
def test_add_layernorm_ragged(policy):
    print(f"\n[gpu] add_layernorm ragged {policy}", flush=True)
    for cols in COLS:
        for rows in (1, 7, 37):
            inp = synth.add_layernorm_inputs(rows, cols, seed=cols + rows, mean=3.0, std=2.0)
            for with_sum, affine in ((True, True), (False, False)):
                st, y, s = run_add(inp, policy, with_sum=with_sum, affine=affine)
                assert st == lr.LR_OK
                check(inp, policy, y, s, affine, f"{rows}x{cols} sum={with_sum} affine={affine}")


@pytest.mark.parametrize("mode", ["y_is_x", "y_is_res", "sum_is_x", "sum_is_res"])
def test_add_layernorm_in_place(mode):
    for rows, cols in [(37, 1537), (64, 6144), (3, 40000)]:
        inp = synth.add_layernorm_inputs(rows, cols, seed=rows)
        for policy in ("unordered_tree", "ordered_fold"):
            st, y, s = run_add(inp, policy, mode=mode)
            assert st == lr.LR_OK
            check(inp, policy, y, s, what=f"{mode} {rows}x{cols} {policy}")


@pytest.mark.parametrize("pads", [(1, 0, 0, 0), (0, 1, 0, 0), (0, 0, 2, 3), (3, 1, 2, 0), (2, 2, 2, 2)])
def test_add_layernorm_misaligned_bases(pads):
    for rows, cols in [(5, 1537), (6, 4096), (2, 12289)]:
        inp = synth.add_layernorm_inputs(rows, cols, seed=sum(pads) + cols)
        for policy in ("unordered_tree", "ordered_fold"):
            st, y, s = run_add(inp, policy, pads=pads)
            assert st == lr.LR_OK
            check(inp, policy, y, s, what=f"pads {pads} {rows}x{cols} {policy}")


def test_add_layernorm_every_legal_plan():
    facts = lr.lr_device_facts_query()
    n = 0
    for rows, cols in [(17, 257), (7, 4096), (3, 12289), (2, 6144)]:
        inp = synth.add_layernorm_inputs(rows, cols, seed=rows * cols)
        for policy in ("unordered_tree", "ordered_fold"):
            plans = lr.lr_plan_enumerate(facts, "add_layernorm", rows, cols, policy, 1 if cols % 4 == 0 else 0)
            print(f"\n[gpu] add_layernorm plans {rows}x{cols} {policy}: {len(plans)}", flush=True)
            for p in plans:
                st, y, s = run_add(inp, policy, plan=p)
                assert st == lr.LR_OK, (p, lr.lr_status_string(st))
                check(inp, policy, y, s, what=f"{rows}x{cols} {p}")
                n += 1
    assert n > 40


def test_add_layernorm_zero_residual_equals_layernorm_on_gpu():
    inp = synth.layernorm_inputs(64, 6144, seed=4)
    x = torch.from_numpy(inp["x"]).to(DEV)
    z = torch.zeros_like(x)
    g, b = dev(inp["gamma"]), dev(inp["beta"])
    y1, y2 = torch.empty_like(x), torch.empty_like(x)
    for policy in ("unordered_tree", "ordered_fold"):
        plan = lr.lr_plan_query("layernorm", 64, 6144, policy)
        lr.check(lr.lr_layernorm_f32(x, g, b, y1, 64, 6144, EPS, policy, plan=plan))
        lr.check(lr.lr_add_layernorm_f32(x, z, g, b, y2, None, 64, 6144, EPS, policy, plan=plan))
        torch.cuda.synchronize()
        # same plan, x + 0 == x: the same FP32 operations in the same order
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)), policy
