"""Sub-wave teams on the GPU (CACHE plans with lanes_per_row 4, 8, 16 or 32:
64 / lanes_per_row rows share one wavefront, "TIRx Metal reduction
lowering", section 4.3 packing taken below the wave).  Every operation, at
narrow widths (1 .. 256 columns, ragged), under every legal sub-wave plan
with one and four waves per workgroup, with a row count that leaves the
last wave and the last workgroup part-empty, rows 4-byte offset from their
16-byte grid, and guard regions around every output.  Results are checked
against the oracle at |gpu - ref| <= 1e-6 + 1e-5 |ref| (row sums against
1e-6 + 1e-5 sum |x|; minimum and maximum exact), and a row's neighbours in
the same wave must not leak into it: alternate rows are scaled by 1e3."""
import numpy as np
import pytest
import torch

import oracle
import row_reductions_amd as lr
import synth
from gpu_util import ATOL, DEV, RTOL, assert_parity, bits_equal, guards_intact, placed

pytestmark = pytest.mark.gpu

OPS = ["softmax", "rmsnorm", "layernorm", "cross_entropy", "add_layernorm", "row_sum", "row_minmax"]
COLS = [1, 2, 3, 4, 5, 7, 8, 16, 17, 31, 33, 64, 65, 100, 128, 129, 200, 256]
ROWS = 157  # leaves part-empty waves and workgroups for every team width
EPS = {"rmsnorm": 1e-6, "layernorm": 1e-5, "add_layernorm": 1e-5}


def narrow_plans(op, cols, aligned):
    facts = lr.lr_device_facts_query()
    return [p for p in lr.lr_plan_enumerate(facts, op, ROWS, cols, "unordered_tree", aligned)
            if p.lanes_per_row < 64 and p.threads_per_block in (64, 256)]


def inputs(op, cols, seed):
    x = synth.normal_f32(seed, 0, ROWS * cols, 0.5, 2.0).reshape(ROWS, cols)
    x[1::2] *= 1e3  # neighbouring rows of very different scale
    d = {"x": x, "gamma": synth.uniform_f32(seed, 1, cols, 0.5, 1.5),
         "beta": synth.normal_f32(seed, 2, cols, 0.0, 0.1),
         "residual": synth.normal_f32(seed, 4, ROWS * cols, 0.0, 1.0).reshape(ROWS, cols)}
    lab = synth.labels_i64(seed, 3, ROWS, 0, cols).copy()
    lab[::11] = -1
    lab[5::13] = cols
    d["labels"] = lab
    return d


@pytest.mark.parametrize("cols", COLS)
@pytest.mark.parametrize("op", OPS)
def test_sub_wave_teams(op, cols):
    d = inputs(op, cols, seed=cols)
    x = d["x"]
    checked = 0
    for off in (0, 1):
        aligned = 1 if off == 0 and cols % 4 == 0 else 0
        # a misaligned 256-column row spans 65 chunks: past the widest team
        for plan in narrow_plans(op, cols, aligned):
            print(f"\n[gpu] narrow {op} {ROWS}x{cols} off={off} lanes={plan.lanes_per_row} "
                  f"Q={plan.rows_per_block} nch={plan.chunks_per_lane}", flush=True)
            xv, _ = placed(x, off)
            g = torch.from_numpy(d["gamma"]).to(DEV)
            b = torch.from_numpy(d["beta"]).to(DEV)
            what = f"{op} {ROWS}x{cols} off={off} {plan}"
            if op in ("cross_entropy", "row_sum", "row_minmax"):
                o1, o2 = placed(np.zeros(ROWS, np.float32), off), placed(np.zeros(ROWS, np.float32), off)
                if op == "cross_entropy":
                    st = lr.lr_cross_entropy_f32(xv, torch.from_numpy(d["labels"]).to(DEV), o1[0], ROWS, cols,
                                                 plan=plan)
                elif op == "row_sum":
                    st = lr.lr_row_sum_f32(xv, o1[0], ROWS, cols, plan=plan)
                else:
                    st = lr.lr_row_minmax_f32(xv, o1[0], o2[0], ROWS, cols, plan=plan)
                torch.cuda.synchronize()
                assert st == lr.LR_OK, lr.lr_status_string(st)
                assert guards_intact(*o1) and guards_intact(*o2), what
                got = o1[0].cpu().numpy()
                if op == "cross_entropy":
                    assert_parity(got, oracle.cross_entropy(x, d["labels"]), what)
                elif op == "row_sum":
                    bound = ATOL + RTOL * np.abs(x.astype(np.float64)).sum(axis=1)
                    assert (np.abs(got - oracle.row_sum(x)) <= bound).all(), what
                else:
                    lo, hi = oracle.row_minmax(x)
                    assert np.array_equal(got, lo) and np.array_equal(o2[0].cpu().numpy(), hi), what
            else:
                yv, yfull = placed(np.zeros_like(x), off)
                if op == "softmax":
                    st = lr.lr_softmax_f32(xv, yv, ROWS, cols, plan=plan)
                    ref = oracle.softmax(x)
                elif op == "rmsnorm":
                    st = lr.lr_rmsnorm_f32(xv, g, yv, ROWS, cols, EPS[op], plan=plan)
                    ref = oracle.rmsnorm(x, d["gamma"], EPS[op])
                elif op == "layernorm":
                    st = lr.lr_layernorm_f32(xv, g, b, yv, ROWS, cols, EPS[op], plan=plan)
                    ref = oracle.layernorm(x, d["gamma"], d["beta"], EPS[op])
                else:
                    rv, _ = placed(d["residual"], off)
                    sv, sfull = placed(np.zeros_like(x), off)
                    st = lr.lr_add_layernorm_f32(xv, rv, g, b, yv, sv, ROWS, cols, EPS[op], plan=plan)
                    ref, comb = oracle.add_layernorm(x, d["residual"], d["gamma"], d["beta"], EPS[op],
                                                     with_sum=True)
                torch.cuda.synchronize()
                assert st == lr.LR_OK, lr.lr_status_string(st)
                assert guards_intact(yv, yfull), what
                assert_parity(yv.cpu().numpy(), ref, what)
                if op == "add_layernorm":
                    assert guards_intact(sv, sfull), what
                    assert np.array_equal(sv.cpu().numpy(), comb), what
            checked += 1
    assert checked >= 1


def test_prior_packs_narrow_rows():
    """many narrow rows: the automatic plan shares each wave between rows;
    few rows or wide rows keep whole waves"""
    facts = lr.lr_device_facts_mi355x()
    p = lr.lr_plan_for_device(facts, "softmax", 262144, 64, "unordered_tree", 1)
    assert p.lanes_per_row == 16 and p.chunks_per_lane == 1
    p = lr.lr_plan_for_device(facts, "rmsnorm", 1 << 20, 16, "unordered_tree", 1)
    assert p.lanes_per_row == 4
    assert lr.lr_plan_for_device(facts, "softmax", 37, 64, "unordered_tree", 1).lanes_per_row == 64 * \
        lr.lr_plan_for_device(facts, "softmax", 37, 64, "unordered_tree", 1).waves_per_row
    assert lr.lr_plan_for_device(facts, "softmax", 262144, 512, "unordered_tree", 1).lanes_per_row == 64


TREE_COLS = [4, 8, 16, 32, 64, 100, 128]  # aligned rows (TREE plans need them)


def replay_ok(op, d, got, what, y2=None):
    """ordered_tree gate: bit-equal FP32 replays (norms, sums), the widened
    bar for softmax / cross-entropy, exact min / max"""
    import math
    x = d["x"]
    pol = "ordered_tree"
    if op == "rmsnorm":
        rep = oracle.rmsnorm_ordered_f32(x, d["gamma"], EPS[op], pol)
    elif op == "layernorm":
        rep = oracle.layernorm_ordered_f32(x, d["gamma"], d["beta"], EPS[op], pol)
    elif op == "add_layernorm":
        _, comb = oracle.add_layernorm(x, d["residual"], None, None, EPS[op], with_sum=True)
        rep = oracle.layernorm_ordered_f32(comb, d["gamma"], d["beta"], EPS[op], pol)
    elif op == "row_sum":
        rep = np.array([oracle.ordered_sum_f32(r, pol) for r in x], dtype=np.float32)
    elif op == "row_minmax":
        lo, hi = oracle.row_minmax(x)
        assert np.array_equal(got, lo) and np.array_equal(y2, hi), what
        return
    else:
        n = x.shape[1]
        steps = max(1, math.ceil(math.log2(n)))
        g = steps * 2.0 ** -24 / (1 - steps * 2.0 ** -24)
        ref = oracle.softmax(x) if op == "softmax" else oracle.cross_entropy(x, d["labels"])
        err = np.abs(got.astype(np.float64) - ref)
        bound = ATOL + (RTOL + g) * np.abs(ref) + (g if op == "cross_entropy" else 0.0)
        assert (err <= bound).all(), f"{what}: worst err/bound {(err / bound).max():.3g}"
        return
    assert np.array_equal(got.view(np.uint32), rep.view(np.uint32)), what


@pytest.mark.parametrize("cols", TREE_COLS)
@pytest.mark.parametrize("op", OPS)
def test_sub_wave_tree_teams(op, cols):
    """ordered_tree on sub-wave teams (one chunk per lane): the FP32 tree over
    the row, bit for bit, whatever the team width"""
    d = inputs(op, cols, seed=100 + cols)
    x = d["x"]
    facts = lr.lr_device_facts_query()
    plans = [p for p in lr.lr_plan_enumerate(facts, op, ROWS, cols, "ordered_tree", 1)
             if p.family == lr.LR_FAMILY_TREE and p.lanes_per_row < 64 and p.threads_per_block in (64, 256)]
    assert plans
    g = torch.from_numpy(d["gamma"]).to(DEV)
    b = torch.from_numpy(d["beta"]).to(DEV)
    for plan in plans:
        print(f"\n[gpu] narrow tree {op} {ROWS}x{cols} lanes={plan.lanes_per_row} Q={plan.rows_per_block}", flush=True)
        xv = torch.from_numpy(x).to(DEV)
        what = f"{op} {ROWS}x{cols} ordered_tree {plan}"
        y2 = None
        if op in ("cross_entropy", "row_sum", "row_minmax"):
            o1, o2 = torch.empty(ROWS, device=DEV), torch.empty(ROWS, device=DEV)
            if op == "cross_entropy":
                st = lr.lr_cross_entropy_f32(xv, torch.from_numpy(d["labels"]).to(DEV), o1, ROWS, cols,
                                             "ordered_tree", plan=plan)
            elif op == "row_sum":
                st = lr.lr_row_sum_f32(xv, o1, ROWS, cols, "ordered_tree", plan=plan)
            else:
                st = lr.lr_row_minmax_f32(xv, o1, o2, ROWS, cols, "ordered_tree", plan=plan)
                y2 = o2
            out = o1
        else:
            out = torch.empty_like(xv)
            if op == "softmax":
                st = lr.lr_softmax_f32(xv, out, ROWS, cols, "ordered_tree", plan=plan)
            elif op == "rmsnorm":
                st = lr.lr_rmsnorm_f32(xv, g, out, ROWS, cols, EPS[op], "ordered_tree", plan=plan)
            elif op == "layernorm":
                st = lr.lr_layernorm_f32(xv, g, b, out, ROWS, cols, EPS[op], "ordered_tree", plan=plan)
            else:
                rv = torch.from_numpy(d["residual"]).to(DEV)
                st = lr.lr_add_layernorm_f32(xv, rv, g, b, out, None, ROWS, cols, EPS[op], "ordered_tree", plan=plan)
        torch.cuda.synchronize()
        assert st == lr.LR_OK, lr.lr_status_string(st)
        replay_ok(op, d, out.cpu().numpy(), what, None if y2 is None else y2.cpu().numpy())


@pytest.mark.parametrize("cols", [4, 64, 100, 256, 300, 1024])
def test_negative_zero_rows_under_ordered_policies(cols):
    """rows of -0.0 (and rows of -0.0 with one +0.0) under every ordered policy
    on every plan family: a tree pads with the exact add identity -0, so its
    sum of negative zeros is -0 at every width and on every plan; a fold
    starts from +0 and gives +0; both equal the FP32 replays bit for bit."""
    rows = 6
    x = np.full((rows, cols), -0.0, np.float32)
    x[1::2, cols // 3] = 0.0
    facts = lr.lr_device_facts_query()
    xv = torch.from_numpy(x).to(DEV)
    neg = np.uint32(0x80000000)
    for pol in ("ordered_tree", "ordered_fold", "fold_right"):
        rep = np.array([oracle.ordered_sum_f32(r, pol) for r in x], dtype=np.float32)
        # the tree keeps -0 for the all-negative-zero rows; a fold from +0 gives +0
        want = np.where(np.arange(rows) % 2 == 0, neg if pol == "ordered_tree" else np.uint32(0), np.uint32(0))
        assert np.array_equal(rep.view(np.uint32), want.astype(np.uint32)), (pol, rep)
        for aligned in ((1, 0) if cols % 4 == 0 else (0,)):
            for plan in lr.lr_plan_enumerate(facts, "row_sum", rows, cols, pol, aligned):
                out = torch.full((rows,), 7.0, device=DEV)
                st = lr.lr_row_sum_f32(xv, out, rows, cols, pol, plan=plan)
                torch.cuda.synchronize()
                assert st == lr.LR_OK
                got = out.cpu().numpy()
                assert np.array_equal(got.view(np.uint32), rep.view(np.uint32)), (pol, cols, plan, got, rep)


LANE_COLS = [3, 4, 8, 17, 20, 32, 48, 50, 63, 64]  # misaligned rows included


def run_op(op, d, cols, policy, plan, rows=ROWS):
    """one call; returns the output rows (and the maxima for row_minmax)"""
    x = torch.from_numpy(d["x"]).to(DEV)
    g, b = torch.from_numpy(d["gamma"]).to(DEV), torch.from_numpy(d["beta"]).to(DEV)
    if op in ("cross_entropy", "row_sum", "row_minmax"):
        o1, o2 = torch.empty(rows, device=DEV), torch.empty(rows, device=DEV)
        if op == "cross_entropy":
            st = lr.lr_cross_entropy_f32(x, torch.from_numpy(d["labels"]).to(DEV), o1, rows, cols, policy, plan=plan)
        elif op == "row_sum":
            st = lr.lr_row_sum_f32(x, o1, rows, cols, policy, plan=plan)
        else:
            st = lr.lr_row_minmax_f32(x, o1, o2, rows, cols, policy, plan=plan)
        torch.cuda.synchronize()
        assert st == lr.LR_OK, lr.lr_status_string(st)
        return o1.cpu().numpy(), o2.cpu().numpy()
    y = torch.empty_like(x)
    if op == "softmax":
        st = lr.lr_softmax_f32(x, y, rows, cols, policy, plan=plan)
    elif op == "rmsnorm":
        st = lr.lr_rmsnorm_f32(x, g, y, rows, cols, EPS[op], policy, plan=plan)
    elif op == "layernorm":
        st = lr.lr_layernorm_f32(x, g, b, y, rows, cols, EPS[op], policy, plan=plan)
    else:
        st = lr.lr_add_layernorm_f32(x, torch.from_numpy(d["residual"]).to(DEV), g, b, y, None, rows, cols, EPS[op],
                                     policy, plan=plan)
    torch.cuda.synchronize()
    assert st == lr.LR_OK, lr.lr_status_string(st)
    return y.cpu().numpy(), None


@pytest.mark.parametrize("cols", LANE_COLS)
@pytest.mark.parametrize("op", OPS)
def test_one_lane_per_row_ordered(op, cols):
    """the ordered policies with one lane per row (narrow rows, any alignment): the
    FP32 replays bit for bit (norms, sums), the widened bar (softmax,
    cross-entropy), exact min / max, and every output bit-identical to the
    one-wave-per-row plan's: the same order and the same functions"""
    d = inputs(op, cols, seed=200 + cols)
    facts = lr.lr_device_facts_query()
    for policy in ("ordered_fold", "fold_right", "ordered_tree"):
        plans = lr.lr_plan_enumerate(facts, op, ROWS, cols, policy, 1 if cols % 4 == 0 else 0)
        lanes = [p for p in plans if p.lanes_per_row == 1]
        wave = next(p for p in plans if p.family == lr.LR_FAMILY_ORDERED and p.lanes_per_row == 64)
        assert lanes, (op, cols, policy)
        ref1, ref2 = run_op(op, d, cols, policy, wave)
        for plan in lanes:
            print(f"\n[gpu] lane rows {op} {ROWS}x{cols} {policy} Q={plan.rows_per_block}", flush=True)
            got1, got2 = run_op(op, d, cols, policy, plan)
            what = f"{op} {ROWS}x{cols} {policy} {plan}"
            assert np.array_equal(got1.view(np.uint32), ref1.view(np.uint32)), what + " vs the wave plan"
            if got2 is not None:
                assert np.array_equal(got2.view(np.uint32), ref2.view(np.uint32)), what
            if policy == "ordered_tree":
                replay_ok(op, d, got1, what, got2)
            elif op in ("rmsnorm", "layernorm", "add_layernorm", "row_sum"):
                x = d["x"]
                if op == "rmsnorm":
                    rep = oracle.rmsnorm_ordered_f32(x, d["gamma"], EPS[op], policy)
                elif op == "layernorm":
                    rep = oracle.layernorm_ordered_f32(x, d["gamma"], d["beta"], EPS[op], policy)
                elif op == "add_layernorm":
                    _, comb = oracle.add_layernorm(x, d["residual"], None, None, EPS[op], with_sum=True)
                    rep = oracle.layernorm_ordered_f32(comb, d["gamma"], d["beta"], EPS[op], policy)
                else:
                    rep = np.array([oracle.ordered_sum_f32(r, policy) for r in x], dtype=np.float32)
                assert np.array_equal(got1.view(np.uint32), rep.view(np.uint32)), what


EDGE_COLS = [16, 50]  # the constant-width body (16 = 4 * 4 floats) and the general one


@pytest.mark.parametrize("cols", EDGE_COLS)
def test_one_lane_per_row_edges(cols):
    """one lane per row under ordered_fold, with input and output rows at
    4-byte offsets from the 16-byte grid, in place, gamma / beta absent, and
    the fused residual LayerNorm's combined output: every output between
    intact guard regions; the norms equal the FP32 replays of the policy
    ("TIRx Metal reduction lowering", section 1, the reduction policies) and
    softmax the one-wave-per-row plan, bit for bit"""
    facts = lr.lr_device_facts_query()
    d = inputs("add_layernorm", cols, seed=300 + cols)
    x, res = d["x"], d["residual"]
    policy = "ordered_fold"

    def plan_of(op, lanes):
        return next(p for p in lr.lr_plan_enumerate(facts, op, ROWS, cols, policy, 0)
                    if p.lanes_per_row == lanes and p.family == lr.LR_FAMILY_ORDERED)

    wave_softmax, _ = run_op("softmax", d, cols, policy, plan_of("softmax", 64))
    for xo, yo, in_place, params in ((1, 3, False, True), (2, 2, True, False), (3, 0, False, False)):
        what = f"{ROWS}x{cols} xo={xo} yo={yo} in_place={in_place} gamma/beta={params}"
        print(f"\n[gpu] lane edges {what}", flush=True)
        g = torch.from_numpy(d["gamma"]).to(DEV) if params else None
        b = torch.from_numpy(d["beta"]).to(DEV) if params else None
        gam, bet = (d["gamma"], d["beta"]) if params else (None, None)

        def out_for(xv, xf):
            return (xv, xf) if in_place else placed(np.zeros_like(x), yo)

        xv, xf = placed(x, xo)
        yv, yf = out_for(xv, xf)
        st = lr.lr_rmsnorm_f32(xv, g, yv, ROWS, cols, EPS["rmsnorm"], policy, plan=plan_of("rmsnorm", 1))
        torch.cuda.synchronize()
        assert st == lr.LR_OK, lr.lr_status_string(st)
        assert guards_intact(yv, yf), "rmsnorm " + what
        bits_equal(yv.cpu().numpy(), oracle.rmsnorm_ordered_f32(x, gam, EPS["rmsnorm"], policy), "rmsnorm " + what)

        xv, xf = placed(x, xo)
        rv, _ = placed(res, xo)
        yv, yf = out_for(xv, xf)
        sv, sf = placed(np.zeros_like(x), yo)
        st = lr.lr_add_layernorm_f32(xv, rv, g, b, yv, sv, ROWS, cols, EPS["add_layernorm"], policy,
                                     plan=plan_of("add_layernorm", 1))
        torch.cuda.synchronize()
        assert st == lr.LR_OK, lr.lr_status_string(st)
        assert guards_intact(yv, yf) and guards_intact(sv, sf), "add_layernorm " + what
        _, comb = oracle.add_layernorm(x, res, None, None, EPS["add_layernorm"], with_sum=True)
        comb = comb.astype(np.float32)
        bits_equal(sv.cpu().numpy(), comb, "add_layernorm sum " + what)
        bits_equal(yv.cpu().numpy(), oracle.layernorm_ordered_f32(comb, gam, bet, EPS["add_layernorm"], policy),
                   "add_layernorm " + what)

        xv, xf = placed(x, xo)
        yv, yf = out_for(xv, xf)
        st = lr.lr_softmax_f32(xv, yv, ROWS, cols, policy, plan=plan_of("softmax", 1))
        torch.cuda.synchronize()
        assert st == lr.LR_OK, lr.lr_status_string(st)
        assert guards_intact(yv, yf), "softmax " + what
        bits_equal(yv.cpu().numpy(), wave_softmax, "softmax vs the wave plan " + what)
