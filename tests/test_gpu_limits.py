"""Limits of the C ABI on the GPU.

The widest row it accepts, cols = 2^24 - 1 (a 64 MiB row), for every
operation under the unordered policy and the ordered ones, and the first width
past the limit, which is rejected before any launch.  Ordered RMSNorm,
LayerNorm and row sums must equal the FP32 replays bit for bit.  For ordered
softmax and cross-entropy the serial-sum error bound is vacuous at this width,
so the reference replays the policy's FP32 sum over the correctly rounded
exponentials (the device's expf is within an ulp or two of them; the sums
then differ by a few ulp at most).

A tall, narrow problem, (2^26 + 3) x 1: under a whole-wave plan (64 lanes per
row) its grid exceeds one dispatch (2^31 work-items), so the call runs as
several dispatches of whole workgroups of rows, and every row, the last
piece's included, must hold its result.  The automatic plan (sub-wave teams,
16 rows per wave) covers it in one dispatch."""
import numpy as np
import pytest
import torch

import oracle
import row_reductions_amd as lr
from gpu_util import DEV, assert_parity, check_output

pytestmark = pytest.mark.gpu

COLS = (1 << 24) - 1
ROWS = 2


@pytest.fixture(scope="module")
def data():
    gen = torch.Generator(device=DEV).manual_seed(24)
    x = torch.randn(ROWS, COLS, device=DEV, generator=gen)
    r = torch.randn(ROWS, COLS, device=DEV, generator=gen)
    g = torch.rand(COLS, device=DEV, generator=gen) + 0.5
    b = torch.randn(COLS, device=DEV, generator=gen) * 0.1
    lab = torch.tensor([COLS - 1, 12345], dtype=torch.int64, device=DEV)
    host = {k: v.cpu().numpy() for k, v in dict(x=x, r=r, g=g, b=b, lab=lab).items()}
    return dict(x=x, r=r, g=g, b=b, lab=lab), host


def replay_softmax_state(x, policy):
    """(row max, FP32 sum of exp(x - max) in the policy's order) per row"""
    m = x.max(axis=1)
    e = np.exp((x - m[:, None]).astype(np.float64)).astype(np.float32)
    s = np.array([oracle.ordered_sum_f32(row, policy) for row in e], dtype=np.float64)
    return m.astype(np.float64), s, e


@pytest.mark.parametrize("policy", ["unordered_tree", "ordered_fold", "ordered_tree"])
@pytest.mark.parametrize("op", ["softmax", "rmsnorm", "layernorm", "cross_entropy", "add_layernorm", "row_sum",
                                "row_minmax"])
def test_widest_row(data, op, policy):
    d, h = data
    plan = lr.lr_plan_query(op, ROWS, COLS, policy)
    print(f"\n[gpu] widest row {op} {ROWS}x{COLS} {policy}: {lr.FAMILY_NAMES[plan.family]}", flush=True)
    eps = {"rmsnorm": 1e-6, "layernorm": 1e-5, "add_layernorm": 1e-5}.get(op)
    if op in ("cross_entropy", "row_sum", "row_minmax"):
        o1, o2 = torch.empty(ROWS, device=DEV), torch.empty(ROWS, device=DEV)
        if op == "cross_entropy":
            st = lr.lr_cross_entropy_f32(d["x"], d["lab"], o1, ROWS, COLS, policy)
        elif op == "row_sum":
            st = lr.lr_row_sum_f32(d["x"], o1, ROWS, COLS, policy)
        else:
            st = lr.lr_row_minmax_f32(d["x"], o1, o2, ROWS, COLS, policy)
        torch.cuda.synchronize()
        assert st == lr.LR_OK, lr.lr_status_string(st)
        got = o1.cpu().numpy()
        if op == "cross_entropy" and policy == "unordered_tree":
            check_output(op, {"logits": h["x"], "labels": h["lab"]}, None, policy, got, "widest row")
        elif op == "cross_entropy":
            m, s, _ = replay_softmax_state(h["x"], policy)
            sel = h["x"][np.arange(ROWS), h["lab"]].astype(np.float64)  # both labels are in range
            assert_parity(got, np.log(s) + m - sel, "widest row, ordered")
        elif op == "row_sum":
            if policy == "unordered_tree":
                ref = oracle.row_sum(h["x"])
                bound = 1e-6 + 1e-5 * np.abs(h["x"].astype(np.float64)).sum(axis=1)
                assert (np.abs(got - ref) <= bound).all(), (got, ref)
            else:
                rep = np.array([oracle.ordered_sum_f32(row, policy) for row in h["x"]], dtype=np.float32)
                assert np.array_equal(got.view(np.uint32), rep.view(np.uint32)), (got, rep)
        else:
            lo, hi = oracle.row_minmax(h["x"])
            assert np.array_equal(got, lo) and np.array_equal(o2.cpu().numpy(), hi)
        return
    y = torch.empty_like(d["x"])
    if op == "softmax":
        st = lr.lr_softmax_f32(d["x"], y, ROWS, COLS, policy)
        inp = {"x": h["x"]}
    elif op == "rmsnorm":
        st = lr.lr_rmsnorm_f32(d["x"], d["g"], y, ROWS, COLS, eps, policy)
        inp = {"x": h["x"], "gamma": h["g"]}
    elif op == "layernorm":
        st = lr.lr_layernorm_f32(d["x"], d["g"], d["b"], y, ROWS, COLS, eps, policy)
        inp = {"x": h["x"], "gamma": h["g"], "beta": h["b"]}
    else:
        st = lr.lr_add_layernorm_f32(d["x"], d["r"], d["g"], d["b"], y, None, ROWS, COLS, eps, policy)
    torch.cuda.synchronize()
    assert st == lr.LR_OK, lr.lr_status_string(st)
    got = y.cpu().numpy()
    if op == "add_layernorm":
        if policy == "unordered_tree":
            assert_parity(got, oracle.add_layernorm(h["x"], h["r"], h["g"], h["b"], eps), "widest row")
        else:
            c = (h["x"] + h["r"]).astype(np.float32)
            rep = oracle.layernorm_ordered_f32(c, h["g"], h["b"], eps, policy)
            assert np.array_equal(got.view(np.uint32), rep.view(np.uint32))
        return
    if op == "softmax" and policy != "unordered_tree":
        _, s, e = replay_softmax_state(h["x"], policy)
        assert_parity(got, e.astype(np.float64) / s[:, None], "widest row, ordered")
        return
    if policy == "ordered_tree" and op in ("rmsnorm", "layernorm"):
        f = oracle.rmsnorm_ordered_f32 if op == "rmsnorm" else oracle.layernorm_ordered_f32
        args = (h["x"], h["g"], eps, policy) if op == "rmsnorm" else (h["x"], h["g"], h["b"], eps, policy)
        rep = f(*args)
        assert np.array_equal(got.view(np.uint32), rep.view(np.uint32))
        return
    check_output(op, inp, eps, policy, got, "widest row")


def test_one_past_the_widest_row_is_rejected():
    x = torch.empty(8, device=DEV)
    st = lr.lr_softmax_f32(x, x, 1, 1 << 24)
    assert st == lr.LR_ERR_INVALID_SHAPE


TALL = (1 << 26) + 3


@pytest.fixture(scope="module")
def tall():
    gen = torch.Generator(device=DEV).manual_seed(26)
    x = torch.randn(TALL, 1, device=DEV, generator=gen)
    lab = torch.zeros(TALL, dtype=torch.int64, device=DEV)
    lab[::997] = 1       # out of range for one column
    lab[::1009] = -1
    return x, lab, x.cpu().numpy(), lab.cpu().numpy()


def whole_wave_plan(op, policy):
    """the automatic plan when it gives each row a whole wave, else (the
    automatic plan packs several rows per wave, or one row per lane) the
    whole-wave CACHE or ORDERED plan with 16 rows per workgroup"""
    plan = lr.lr_plan_query(op, TALL, 1, policy)
    if plan.lanes_per_row == 64:
        return plan
    facts = lr.lr_device_facts_query()
    return next(p for p in lr.lr_plan_enumerate(facts, op, TALL, 1, policy, 0)
                if p.family in (lr.LR_FAMILY_CACHE, lr.LR_FAMILY_ORDERED) and p.lanes_per_row == 64
                and p.rows_per_block == 16)


@pytest.mark.parametrize("op,policy", [(o, "unordered_tree") for o in
                                       ("softmax", "rmsnorm", "layernorm", "cross_entropy", "add_layernorm",
                                        "row_sum", "row_minmax")]
                         + [("row_sum", "ordered_fold"), ("rmsnorm", "ordered_tree"), ("softmax", "fold_right"),
                            ("softmax", "automatic"), ("layernorm", "automatic")])
def test_tall_narrow_problem_runs_as_several_dispatches(tall, op, policy):
    x, lab, hx, hlab = tall
    auto = policy == "automatic"
    policy = "unordered_tree" if auto else policy
    plan = lr.lr_plan_query(op, TALL, 1, policy) if auto else whole_wave_plan(op, policy)
    step = lr.lr_dispatch_rows(plan, TALL)
    print(f"\n[gpu] tall {op} {TALL}x1 {policy}: {lr.FAMILY_NAMES[plan.family]} lanes={plan.lanes_per_row} "
          f"Q={plan.rows_per_block}, {-(-TALL // step)} dispatches", flush=True)
    assert step == TALL if auto else step < TALL
    nan = float("nan")
    if op in ("cross_entropy", "row_sum", "row_minmax"):
        o1, o2 = torch.full((TALL,), nan, device=DEV), torch.full((TALL,), nan, device=DEV)
        if op == "cross_entropy":
            st = lr.lr_cross_entropy_f32(x, lab, o1, TALL, 1, policy, plan=plan)
        elif op == "row_sum":
            st = lr.lr_row_sum_f32(x, o1, TALL, 1, policy, plan=plan)
        else:
            st = lr.lr_row_minmax_f32(x, o1, o2, TALL, 1, policy, plan=plan)
        torch.cuda.synchronize()
        assert st == lr.LR_OK, lr.lr_status_string(st)
        got = o1.cpu().numpy()
        if op == "cross_entropy":
            assert_parity(got, oracle.cross_entropy(hx, hlab), "tall")
        elif op == "row_sum":
            assert np.array_equal(got, hx[:, 0])  # a one-element sum is exact
        else:
            lo, hi = oracle.row_minmax(hx)
            assert np.array_equal(got, lo) and np.array_equal(o2.cpu().numpy(), hi)
        return
    y = torch.full_like(x, nan)
    g = torch.full((1,), 1.5, device=DEV)
    b = torch.full((1,), 0.25, device=DEV)
    if op == "softmax":
        st = lr.lr_softmax_f32(x, y, TALL, 1, policy, plan=plan)
        ref = np.ones((TALL, 1))
    elif op == "rmsnorm":
        st = lr.lr_rmsnorm_f32(x, g, y, TALL, 1, 1e-6, policy, plan=plan)
        ref = oracle.rmsnorm(hx, np.array([1.5], np.float32), 1e-6)
    elif op == "layernorm":
        st = lr.lr_layernorm_f32(x, g, b, y, TALL, 1, 1e-5, policy, plan=plan)
        ref = np.full((TALL, 1), 0.25)  # a one-column row has zero variance: y = beta
    else:
        st = lr.lr_add_layernorm_f32(x, x, g, b, y, None, TALL, 1, 1e-5, policy, plan=plan)
        ref = np.full((TALL, 1), 0.25)
    torch.cuda.synchronize()
    assert st == lr.LR_OK, lr.lr_status_string(st)
    assert_parity(y.cpu().numpy(), ref, f"tall {op}")
