"""GPU parity of the standalone row reductions through the C ABI: row sum
and row minimum/maximum together ("TIRx Metal reduction lowering",
section 8: row sums at widths 127, 257, 1024 and 4096, minimum and maximum
at 7 x 1024).

Row minimum and maximum are input values, so every policy and plan must
return them exactly.  Row sums: ordered_fold must equal the CPU FP32 left
fold bit for bit; unordered_tree sums are compared with the double oracle
under |gpu - ref| <= 1e-6 + 1e-5 * sum_j |x_j| -- the stated relative bar
taken on the sum's own scale, since an FP32 sum in any order errs in
proportion to sum |x_j|, not to the (possibly cancelled) result -- and, on
positive data, under the plain bar 1e-6 + 1e-5 |ref|."""
import numpy as np
import pytest
import torch

import oracle
import row_reductions_amd as lr
import synth
from gpu_util import DEV, workspace_for

pytestmark = pytest.mark.gpu


def place(a, pad=0):
    rows, cols = a.shape
    full = torch.empty(rows * cols + pad + 8, dtype=torch.float32, device=DEV)
    v = full[pad:pad + rows * cols].view(rows, cols)
    v.copy_(torch.from_numpy(np.ascontiguousarray(a)).to(DEV))
    return v


def gpu_sum(x, policy, plan=None, pad=0):
    rows, cols = x.shape
    xv = place(x, pad)
    out = torch.full((rows,), float("nan"), device=DEV)
    st = lr.lr_row_sum_f32(xv, out, rows, cols, policy, plan=plan, workspace=workspace_for(plan, rows))
    torch.cuda.synchronize()
    return st, out.cpu().numpy()


def gpu_minmax(x, policy, plan=None, pad=0, want=(True, True)):
    rows, cols = x.shape
    xv = place(x, pad)
    lo = torch.full((rows,), float("nan"), device=DEV) if want[0] else None
    hi = torch.full((rows,), float("nan"), device=DEV) if want[1] else None
    st = lr.lr_row_minmax_f32(xv, lo, hi, rows, cols, policy, plan=plan, workspace=workspace_for(plan, rows))
    torch.cuda.synchronize()
    return st, (lo.cpu().numpy() if lo is not None else None), (hi.cpu().numpy() if hi is not None else None)


def check_sum(x, got, policy, what, positive=False):
    if policy == "ordered_fold":
        rep = np.array([oracle.fold_left_f32(row) for row in x], dtype=np.float32)
        assert np.array_equal(got.view(np.uint32), rep.view(np.uint32)), f"{what}: differs from the FP32 fold"
        return
    ref = oracle.row_sum(x)
    err = np.abs(got.astype(np.float64) - ref)
    scale = np.abs(ref) if positive else np.abs(x.astype(np.float64)).sum(axis=1)
    bound = 1e-6 + 1e-5 * scale
    assert (err <= bound).all(), f"{what}: worst err/bound {(err / bound).max():.3g}"


def check_minmax(x, lo, hi, what):
    rlo, rhi = oracle.row_minmax(x)
    if lo is not None:
        assert np.array_equal(lo, rlo), f"{what}: min"
    if hi is not None:
        assert np.array_equal(hi, rhi), f"{what}: max"


PAGE_WIDTHS = [127, 257, 1024, 4096]
RAGGED = [1, 2, 3, 4, 5, 63, 64, 65, 255, 256, 1537, 6144, 12289, 32000, 40001]


@pytest.mark.parametrize("policy", ["unordered_tree", "ordered_fold"])
def test_row_sum_page_widths_and_ragged(policy):
    print(f"\n[gpu] row sum widths {policy}", flush=True)
    for cols in PAGE_WIDTHS + RAGGED:
        for rows in (1, 7, 37):
            x = synth.normal_f32(cols, 0, rows * cols, 0.5, 2.0).reshape(rows, cols)
            st, got = gpu_sum(x, policy)
            assert st == lr.LR_OK
            check_sum(x, got, policy, f"{rows}x{cols}")
            xp = synth.uniform_f32(cols + 1, 0, rows * cols, 0.5, 1.5).reshape(rows, cols)
            st, got = gpu_sum(xp, policy)
            check_sum(xp, got, policy, f"positive {rows}x{cols}", positive=True)


@pytest.mark.parametrize("policy", ["unordered_tree", "ordered_fold"])
def test_row_minmax_7x1024_and_ragged(policy):
    print(f"\n[gpu] row minmax {policy}", flush=True)
    for rows, cols in [(7, 1024)] + [(r, c) for c in PAGE_WIDTHS + RAGGED for r in (1, 5, 37)]:
        x = synth.normal_f32(rows * 31 + cols, 0, rows * cols, 0.0, 10.0).reshape(rows, cols)
        st, lo, hi = gpu_minmax(x, policy)
        assert st == lr.LR_OK
        check_minmax(x, lo, hi, f"{rows}x{cols}")


def test_row_minmax_extremes_at_row_ends_and_one_output():
    x = synth.normal_f32(3, 0, 9 * 4099, 0.0, 1.0).reshape(9, 4099)
    x[:, 0] = -100.0
    x[:, -1] = 100.0
    x[4, 0], x[4, -1] = 200.0, -200.0
    for policy in ("unordered_tree", "ordered_fold"):
        for want in ((True, True), (True, False), (False, True)):
            for pad in (0, 1, 3):
                st, lo, hi = gpu_minmax(x, policy, pad=pad, want=want)
                assert st == lr.LR_OK
                check_minmax(x, lo, hi, f"ends {policy} {want} pad {pad}")


def test_row_sum_misaligned_bases():
    for pad in (1, 2, 3):
        for rows, cols in [(5, 1537), (6, 4096), (2, 12289)]:
            x = synth.normal_f32(pad + cols, 0, rows * cols, 0.0, 1.0).reshape(rows, cols)
            for policy in ("unordered_tree", "ordered_fold"):
                st, got = gpu_sum(x, policy, pad=pad)
                assert st == lr.LR_OK
                check_sum(x, got, policy, f"pad {pad} {rows}x{cols}")


@pytest.mark.parametrize("op", ["row_sum", "row_minmax"])
def test_every_legal_plan(op):
    facts = lr.lr_device_facts_query()
    n = 0
    for rows, cols in [(17, 257), (7, 4096), (3, 12289), (5, 64), (2, 6144)]:
        x = synth.normal_f32(rows + cols, 0, rows * cols, 0.25, 3.0).reshape(rows, cols)
        for policy in ("unordered_tree", "ordered_fold"):
            plans = lr.lr_plan_enumerate(facts, op, rows, cols, policy, 1 if cols % 4 == 0 else 0)
            print(f"\n[gpu] {op} plans {rows}x{cols} {policy}: {len(plans)}", flush=True)
            for p in plans:
                if op == "row_sum":
                    st, got = gpu_sum(x, policy, plan=p)
                    assert st == lr.LR_OK, (p, lr.lr_status_string(st))
                    check_sum(x, got, policy, f"{rows}x{cols} {p}")
                else:
                    st, lo, hi = gpu_minmax(x, policy, plan=p)
                    assert st == lr.LR_OK, (p, lr.lr_status_string(st))
                    check_minmax(x, lo, hi, f"{rows}x{cols} {p}")
                n += 1
    assert n > 40


def test_row_reductions_full_size_4096x32000():
    # the cross-entropy workload's logits shape
    inp = synth.cross_entropy_inputs(4096, 32000, seed=0)
    x = inp["logits"]
    xv = torch.from_numpy(x).to(DEV)
    s = torch.empty(4096, device=DEV)
    lo, hi = torch.empty(4096, device=DEV), torch.empty(4096, device=DEV)
    for policy in ("unordered_tree", "ordered_fold"):
        print(f"\n[gpu] row reductions 4096x32000 {policy}", flush=True)
        lr.check(lr.lr_row_sum_f32(xv, s, 4096, 32000, policy))
        lr.check(lr.lr_row_minmax_f32(xv, lo, hi, 4096, 32000, policy))
        torch.cuda.synchronize()
        if policy == "ordered_fold":
            # sampled rows against the FP32 fold (the full replay is slow in Python loops)
            idx = np.arange(0, 4096, 97)
            rep = np.array([oracle.fold_left_f32(x[i]) for i in idx], dtype=np.float32)
            assert np.array_equal(s.cpu().numpy()[idx].view(np.uint32), rep.view(np.uint32))
        else:
            check_sum(x, s.cpu().numpy(), policy, "4096x32000")
        check_minmax(x, lo.cpu().numpy(), hi.cpu().numpy(), "4096x32000")


def test_unordered_row_sum_is_repeatable():
    x = synth.normal_f32(9, 0, 64 * 6144, 0.0, 1.0).reshape(64, 6144)
    _, first = gpu_sum(x, "unordered_tree")
    for _ in range(10):
        _, again = gpu_sum(x, "unordered_tree")
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
