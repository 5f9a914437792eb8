"""Seeded random parity sweep on the GPU: each case draws an operation, a
reduction policy, a ragged shape (cols log-uniform in 1 .. 20000), a plan
(the automatic one, or any legal plan of lr_plan_enumerate, split-row plans
with a workspace of their own), 4-byte offsets of the input and output rows
from their 16-byte grid, an in-place call, optional gamma / beta (each at a
4-byte offset of its own from the grid) and, for
cross-entropy, labels out of range.  Every output sits between guard regions
that must survive.  Gates ("TIRx Metal reduction lowering", section 1, the
reduction policies):
  unordered_tree  |gpu - ref| <= 1e-6 + 1e-5 |ref| against the double oracle
                  (row sums: 1e-6 + 1e-5 sum |x|; LayerNorm rows whose mean
                  exceeds 8 standard deviations add the FP32 rounding of
                  the mean, layernorm_bar);
  ordered ones    RMSNorm, LayerNorm, the fused residual LayerNorm and row
                  sums equal the CPU FP32 replay of the policy bit for bit;
                  softmax and cross-entropy (the device's exp/log) lie within
                  the bar widened by the sum's rounding bound;
  row min / max   exact under every policy.
Each case prints its descriptor before it runs."""
import math

import numpy as np
import pytest
import torch

import oracle
import row_reductions_amd as lr
import synth
from gpu_util import ATOL, DEV, RTOL, assert_parity, bits_equal, guards_intact, placed

pytestmark = pytest.mark.gpu

OPS = ["softmax", "rmsnorm", "layernorm", "cross_entropy", "add_layernorm", "row_sum", "row_minmax"]
POLICIES = ["unordered_tree", "ordered_fold", "ordered_tree", "fold_right"]
EPS = {"rmsnorm": 1e-6, "layernorm": 1e-5, "add_layernorm": 1e-5}
CASES = 640


def draw(k):
    """The k-th case: everything from one seeded generator."""
    g = np.random.default_rng(1000 + k)
    op = OPS[k % len(OPS)]
    policy = POLICIES[(k // len(OPS)) % len(POLICIES)]
    cols = int(round(math.exp(g.uniform(0.0, math.log(20000)))))
    rows = int(g.integers(1, max(2, min(200, 1_500_000 // cols))))
    xo = int(g.integers(0, 4))
    yo = int(g.integers(0, 4))
    in_place = op in ("softmax", "rmsnorm", "layernorm", "add_layernorm") and g.random() < 0.2
    use_plan = g.random() < 0.6
    pick = float(g.random())
    has_g = g.random() < 0.7
    has_b = g.random() < 0.7
    with_sum = op == "add_layernorm" and g.random() < 0.5
    go = int(g.integers(0, 4))  # drawn last: the earlier draws keep their values
    bo = int(g.integers(0, 4))
    return dict(op=op, policy=policy, rows=rows, cols=cols, xo=xo, yo=0 if in_place else yo, in_place=in_place,
                use_plan=use_plan, pick=pick, has_g=has_g, has_b=has_b, with_sum=with_sum, go=go, bo=bo, seed=k)


def inputs(c):
    op, rows, cols, s = c["op"], c["rows"], c["cols"], c["seed"]
    if op == "cross_entropy":
        d = synth.cross_entropy_inputs(rows, cols, seed=s)
        lab = d["labels"].copy()
        g = np.random.default_rng(s)
        for r in g.choice(rows, size=min(rows, 3), replace=False):
            lab[r] = [-1, cols, 1 << 40][int(g.integers(0, 3))]
        d["labels"] = lab
        return d
    if op == "add_layernorm":
        d = synth.add_layernorm_inputs(rows, cols, seed=s, mean=3.0, std=2.0)
    elif op == "layernorm":
        d = synth.layernorm_inputs(rows, cols, seed=s, mean=3.0, std=2.0)
    elif op == "rmsnorm":
        d = synth.rmsnorm_inputs(rows, cols, seed=s)
    elif op == "softmax":
        d = synth.softmax_inputs(rows, cols, seed=s, std=4.0)
    else:
        d = {"x": synth.normal_f32(s, 0, rows * cols, 0.5, 3.0).reshape(rows, cols)}
    if not c["has_g"]:
        d.pop("gamma", None)
    if not c["has_b"]:
        d.pop("beta", None)
    return d


def choose_plan(c, aligned):
    if not c["use_plan"]:
        return None
    facts = lr.lr_device_facts_query()
    plans = lr.lr_plan_enumerate(facts, c["op"], c["rows"], c["cols"], c["policy"], aligned)
    return plans[min(len(plans) - 1, int(c["pick"] * len(plans)))]


def layernorm_bar(x, gam, eps, ref):
    """The parity bar of an unordered LayerNorm, per element.  Rows whose
    mean lies within 8 of their standard deviations of zero keep the stated
    bar 1e-6 + 1e-5 |ref|.  On other rows (a large mean over a small spread:
    two nearly equal values, say) the FP32 two-pass method ("TIRx Metal
    reduction lowering", section 5.1) carries the rounding of the mean into
    every centred value, whatever the kernel: an FP32 sum of n values in any
    order of depth at most D = ceil(n / 64) + 14 (a lane's serial run, then
    trees over lanes and waves) is off by at most D u sum|x|, so the mean by
    D u mean|x|, and each output by that times r |gamma|, r = 1 / sqrt(var +
    eps); those rows get that term on top."""
    xd = x.astype(np.float64)
    n = x.shape[1]
    mu = xd.mean(axis=1, keepdims=True)
    var = ((xd - mu) ** 2).mean(axis=1, keepdims=True)
    bar = ATOL + RTOL * np.abs(ref)
    ill = np.abs(mu) > 8.0 * np.sqrt(var)
    depth = math.ceil(n / 64) + 14
    term = depth * 2.0 ** -24 * np.abs(xd).mean(axis=1, keepdims=True) / np.sqrt(var + eps)
    term = term * (np.abs(gam.astype(np.float64)) if gam is not None else 1.0)
    return bar + np.where(ill, term, 0.0)


def assert_layernorm(got, ref, x, gam, eps, what):
    err = np.abs(got.astype(np.float64) - ref)
    bound = layernorm_bar(x, gam, eps, ref)
    if not (err <= bound).all():
        i = np.unravel_index(np.argmax(err / bound), ref.shape)
        raise AssertionError(f"{what}: parity fails at {i}: gpu={got[i]!r} ref={ref[i]!r} "
                             f"(worst err/bound {(err / bound).max():.3g})")


def ordered_bound(op, policy, n):
    steps = max(1, math.ceil(math.log2(n))) if policy == "ordered_tree" else max(1, n - 1)
    return steps * 2.0 ** -24 / (1 - steps * 2.0 ** -24)


@pytest.mark.parametrize("k", range(CASES))
def test_random_case(k):
    c = draw(k)
    op, policy, rows, cols = c["op"], c["policy"], c["rows"], c["cols"]
    d = inputs(c)
    x = d["logits"] if op == "cross_entropy" else d["x"]
    aligned = 1 if c["xo"] == 0 and cols % 4 == 0 else 0
    plan = choose_plan(c, aligned)
    ws = None
    if plan is not None and plan.family == lr.LR_FAMILY_SPLIT:
        ws = torch.full((lr.lr_plan_workspace_bytes(plan, rows),), 0xFF, dtype=torch.uint8, device=DEV)
    print(f"\n[gpu] fuzz {k}: {op} {rows}x{cols} {policy} xo={c['xo']} yo={c['yo']} in_place={c['in_place']} "
          f"gamma={'gamma' in d}+{c['go']} beta={'beta' in d}+{c['bo']} sum={c['with_sum']} plan={plan}", flush=True)
    xv, xfull = placed(x, c["xo"])
    dv = {"labels": torch.from_numpy(np.ascontiguousarray(d["labels"])).to(DEV) if "labels" in d else None}
    params = {}  # gamma / beta at their drawn 4-byte offsets, between guards that must survive
    for n, off in (("gamma", c["go"]), ("beta", c["bo"])):
        params[n] = placed(d[n], off) if n in d else (None, None)
        dv[n] = params[n][0]
    outs = []  # (view, full buffer) of each output, guards checked below
    if op in ("cross_entropy", "row_sum", "row_minmax"):
        o1 = placed(np.zeros(rows, np.float32), c["yo"])
        o2 = placed(np.zeros(rows, np.float32), c["yo"])
        outs = [o1] + ([o2] if op == "row_minmax" else [])
        if op == "cross_entropy":
            st = lr.lr_cross_entropy_f32(xv, dv["labels"], o1[0], rows, cols, policy, plan=plan, workspace=ws)
        elif op == "row_sum":
            st = lr.lr_row_sum_f32(xv, o1[0], rows, cols, policy, plan=plan, workspace=ws)
        else:
            st = lr.lr_row_minmax_f32(xv, o1[0], o2[0], rows, cols, policy, plan=plan, workspace=ws)
    else:
        yv = xv if c["in_place"] else None
        if yv is None:
            yv, yfull = placed(np.zeros_like(x), c["yo"])
            outs.append((yv, yfull))
        eps = EPS.get(op)
        if op == "softmax":
            st = lr.lr_softmax_f32(xv, yv, rows, cols, policy, plan=plan, workspace=ws)
        elif op == "rmsnorm":
            st = lr.lr_rmsnorm_f32(xv, dv["gamma"], yv, rows, cols, eps, policy, plan=plan, workspace=ws)
        elif op == "layernorm":
            st = lr.lr_layernorm_f32(xv, dv["gamma"], dv["beta"], yv, rows, cols, eps, policy, plan=plan,
                                     workspace=ws)
        else:
            rv, _ = placed(d["residual"], c["xo"])
            sv = None
            if c["with_sum"]:
                sv, sfull = placed(np.zeros_like(x), c["yo"])
                outs.append((sv, sfull))
            st = lr.lr_add_layernorm_f32(xv, rv, dv["gamma"], dv["beta"], yv, sv, rows, cols, eps, policy,
                                         plan=plan, workspace=ws)
        if c["in_place"]:
            outs.insert(0, (xv, xfull))
    torch.cuda.synchronize()
    assert st == lr.LR_OK, lr.lr_status_string(st)
    for view, full in outs:
        assert guards_intact(view, full), f"case {k}: guard written"
    for n, (view, full) in params.items():
        if view is not None:
            assert guards_intact(view, full), f"case {k}: {n} guard written"
            assert np.array_equal(view.cpu().numpy().view(np.uint32), d[n].view(np.uint32)), f"case {k}: {n} written"
    got = [v.cpu().numpy() for v, _ in outs]
    what = f"case {k} {op} {rows}x{cols} {policy}"
    gam, bet = d.get("gamma"), d.get("beta")
    if op == "row_minmax":
        lo, hi = oracle.row_minmax(x)
        assert np.array_equal(got[0], lo) and np.array_equal(got[1], hi), what
        return
    if op == "add_layernorm":
        ref, comb = oracle.add_layernorm(x, d["residual"], gam, bet, EPS[op], with_sum=True)
        if c["with_sum"]:
            bits_equal(got[1], comb.astype(np.float32), what + " sum_out")
        if policy == "unordered_tree":
            assert_layernorm(got[0], ref, comb, gam, EPS[op], what)
        else:
            bits_equal(got[0], oracle.layernorm_ordered_f32(comb, gam, bet, EPS[op], policy), what)
        return
    if op == "row_sum":
        if policy == "unordered_tree":
            bound = ATOL + RTOL * np.abs(x.astype(np.float64)).sum(axis=1)
            assert (np.abs(got[0] - oracle.row_sum(x)) <= bound).all(), what
        else:
            bits_equal(got[0], np.array([oracle.ordered_sum_f32(r, policy) for r in x], dtype=np.float32), what)
        return
    if op in ("rmsnorm", "layernorm") and policy != "unordered_tree":
        rep = (oracle.rmsnorm_ordered_f32(x, gam, EPS[op], policy) if op == "rmsnorm"
               else oracle.layernorm_ordered_f32(x, gam, bet, EPS[op], policy))
        bits_equal(got[0], rep, what)
        return
    if op == "softmax":
        ref = oracle.softmax(x)
    elif op == "cross_entropy":
        ref = oracle.cross_entropy(x, d["labels"])
    elif op == "rmsnorm":
        ref = oracle.rmsnorm(x, gam, EPS[op])
    else:
        ref = oracle.layernorm(x, gam, bet, EPS[op])
    if policy == "unordered_tree":
        if op == "layernorm":
            assert_layernorm(got[0], ref, x, gam, EPS[op], what)
        else:
            assert_parity(got[0], ref, what)
        return
    g = ordered_bound(op, policy, cols)
    err = np.abs(got[0].astype(np.float64) - ref)
    bound = ATOL + (RTOL + g) * np.abs(ref) + (g if op == "cross_entropy" else 0.0)
    assert (err <= bound).all(), f"{what}: worst err/bound {(err / bound).max():.3g}"


def test_cases_cover_every_op_policy_and_plan_kind():
    """the draw spans every (op, policy) pair, split plans, in-place calls
    and misaligned rows"""
    cs = [draw(k) for k in range(CASES)]
    assert {(c["op"], c["policy"]) for c in cs} == {(o, p) for o in OPS for p in POLICIES}
    assert sum(c["in_place"] for c in cs) >= 5 and sum(c["xo"] != 0 for c in cs) >= 50
    assert sum(c["use_plan"] for c in cs) >= 60
