"""GPU checks of the ordered_tree and fold_right policies ("TIRx Metal
reduction lowering", section 1: each reduction carries its ReductionPolicy;
an ordered tree or fold stays ordered).

ordered_tree is the pairwise tree in index order over the contributions
padded with -0.0f to the next power of two; fold_right is the FP32 chain from
the right end.  RMSNorm, LayerNorm, the fused residual LayerNorm and the row
sum have exactly one FP32 result under each: the GPU must equal the CPU FP32
replay (oracle) bit for bit, under every legal plan -- TREE-family plans
(the cache layout) and ORDERED-family plans (one wave per row) alike.
Softmax and cross-entropy use the device's precise exp/log, so they are
checked against the double oracle with the bar widened by the sum's error
bound (log2 n roundings for the tree, n - 1 for the fold), and must still be
bit-identical across plans.  Row minimum and maximum are exact."""
import math

import numpy as np
import pytest
import torch

import oracle
import row_reductions_amd as lr
import synth
from gpu_util import ATOL, DEV, RTOL, dev

pytestmark = pytest.mark.gpu

POLS = ["ordered_tree", "fold_right"]
EPS = {"rmsnorm": 1e-6, "layernorm": 1e-5, "add_layernorm": 1e-5}


def inputs(op, rows, cols, seed):
    if op == "cross_entropy":
        return synth.cross_entropy_inputs(rows, cols, seed=seed)
    if op == "add_layernorm":
        return synth.add_layernorm_inputs(rows, cols, seed=seed, mean=3.0, std=2.0)
    if op == "layernorm":
        return synth.layernorm_inputs(rows, cols, seed=seed, mean=3.0, std=2.0)
    if op == "rmsnorm":
        return synth.rmsnorm_inputs(rows, cols, seed=seed)
    if op == "softmax":
        return synth.softmax_inputs(rows, cols, seed=seed, std=4.0)
    return {"x": synth.normal_f32(seed, 0, rows * cols, 0.5, 3.0).reshape(rows, cols)}


def run(op, inp, policy, plan=None):
    x = inp["logits"] if op == "cross_entropy" else inp["x"]
    rows, cols = x.shape
    xv = dev(x)
    if op == "cross_entropy":
        out = torch.empty(rows, device=DEV)
        st = lr.lr_cross_entropy_f32(xv, dev(inp["labels"]), out, rows, cols, policy, plan=plan)
    elif op == "row_sum":
        out = torch.empty(rows, device=DEV)
        st = lr.lr_row_sum_f32(xv, out, rows, cols, policy, plan=plan)
    elif op == "row_minmax":
        lo, hi = torch.empty(rows, device=DEV), torch.empty(rows, device=DEV)
        st = lr.lr_row_minmax_f32(xv, lo, hi, rows, cols, policy, plan=plan)
        out = torch.stack([lo, hi], 1)
    else:
        out = torch.empty(rows, cols, device=DEV)
        if op == "softmax":
            st = lr.lr_softmax_f32(xv, out, rows, cols, policy, plan=plan)
        elif op == "rmsnorm":
            st = lr.lr_rmsnorm_f32(xv, dev(inp.get("gamma")), out, rows, cols, EPS[op], policy, plan=plan)
        elif op == "layernorm":
            st = lr.lr_layernorm_f32(xv, dev(inp.get("gamma")), dev(inp.get("beta")), out, rows, cols, EPS[op],
                                     policy, plan=plan)
        else:
            st = lr.lr_add_layernorm_f32(xv, dev(inp["residual"]), dev(inp.get("gamma")), dev(inp.get("beta")),
                                         out, None, rows, cols, EPS[op], policy, plan=plan)
    torch.cuda.synchronize()
    assert st == lr.LR_OK, lr.lr_status_string(st)
    return out.cpu().numpy()


def check(op, inp, policy, got, what):
    if op == "rmsnorm":
        rep = oracle.rmsnorm_ordered_f32(inp["x"], inp.get("gamma"), EPS[op], policy)
    elif op == "layernorm":
        rep = oracle.layernorm_ordered_f32(inp["x"], inp.get("gamma"), inp.get("beta"), EPS[op], policy)
    elif op == "add_layernorm":
        _, c = oracle.add_layernorm(inp["x"], inp["residual"], None, None, EPS[op], with_sum=True)
        rep = oracle.layernorm_ordered_f32(c, inp.get("gamma"), inp.get("beta"), EPS[op], policy)
    elif op == "row_sum":
        rep = np.array([oracle.ordered_sum_f32(r, policy) for r in inp["x"]], dtype=np.float32)
    elif op == "row_minmax":
        lo, hi = oracle.row_minmax(inp["x"])
        rep = np.stack([lo, hi], 1)
    else:
        x = inp["logits"] if op == "cross_entropy" else inp["x"]
        n = x.shape[1]
        steps = max(1, math.ceil(math.log2(n))) if policy == "ordered_tree" else max(1, n - 1)
        g = steps * 2.0 ** -24 / (1 - steps * 2.0 ** -24)
        ref = oracle.softmax(x) if op == "softmax" else oracle.cross_entropy(x, inp["labels"])
        err = np.abs(got.astype(np.float64) - ref)
        bound = ATOL + (RTOL + g) * np.abs(ref) + (g if op == "cross_entropy" else 0.0)
        assert (err <= bound).all(), f"{what}: worst err/bound {(err / bound).max():.3g}"
        return
    if not np.array_equal(got.view(np.uint32), rep.view(np.uint32)):
        bad = tuple(np.argwhere(got.view(np.uint32) != rep.view(np.uint32))[0])
        raise AssertionError(f"{what}: differs from the FP32 replay at {bad}: {got[bad]!r} vs {rep[bad]!r}")


OPS = ["softmax", "rmsnorm", "layernorm", "cross_entropy", "add_layernorm", "row_sum", "row_minmax"]
COLS = [1, 2, 3, 4, 5, 63, 64, 65, 127, 255, 256, 257, 1023, 1024, 1537, 4096, 6144, 12289, 32768, 32772, 40000]


@pytest.mark.parametrize("policy", POLS)
@pytest.mark.parametrize("op", OPS)
def test_policy_ragged_sweep(op, policy):
    print(f"\n[gpu] {op} {policy} ragged", flush=True)
    for cols in COLS:
        for rows in (1, 7, 37):
            inp = inputs(op, rows, cols, seed=cols * 7 + rows)
            got = run(op, inp, policy)
            check(op, inp, policy, got, f"{op} {policy} {rows}x{cols}")


@pytest.mark.parametrize("op", OPS)
def test_ordered_tree_every_plan_same_bits(op):
    """every TREE and ORDERED plan gives the replay's bits (and one another's)"""
    facts = lr.lr_device_facts_query()
    n = 0
    for rows, cols in [(17, 256), (7, 4096), (3, 6144), (5, 1000), (2, 32768), (3, 12289)]:
        inp = inputs(op, rows, cols, seed=rows + cols)
        first = None
        for policy in POLS:
            plans = lr.lr_plan_enumerate(facts, op, rows, cols, policy, 1 if cols % 4 == 0 else 0)
            fams = sorted({p.family for p in plans})
            print(f"\n[gpu] {op} {rows}x{cols} {policy}: {len(plans)} plans, families {fams}", flush=True)
            first = None
            for p in plans:
                got = run(op, inp, policy, plan=p)
                check(op, inp, policy, got, f"{op} {rows}x{cols} {policy} {p}")
                if first is None:
                    first = got
                assert np.array_equal(got.view(np.uint32), first.view(np.uint32)), (op, policy, p)
                n += 1
    assert n > 40


def test_policies_are_observable():
    # the same data under fold_left, ordered_tree and fold_right gives three
    # different LayerNorm results (the order is real, not a relabelling)
    inp = inputs("layernorm", 16, 6144, seed=1)
    outs = [run("layernorm", inp, pol) for pol in ("ordered_fold", "ordered_tree", "fold_right")]
    for i in range(3):
        for j in range(i + 1, 3):
            assert not np.array_equal(outs[i], outs[j])


@pytest.mark.parametrize("name,op", [("softmax_768x6144", "softmax"), ("rmsnorm_768x6144", "rmsnorm"),
                                     ("layernorm_768x6144", "layernorm"), ("rmsnorm_256x3072", "rmsnorm")])
def test_workloads_under_ordered_tree(name, op):
    inp = synth.workload_inputs(name)
    for policy in POLS:
        print(f"\n[gpu] {name} {policy}", flush=True)
        got = run(op, inp, policy)
        check(op, inp, policy, got, f"{name} {policy}")


def test_ordered_tree_repeatable():
    inp = inputs("softmax", 64, 6144, seed=3)
    first = run("softmax", inp, "ordered_tree")
    for _ in range(10):
        assert np.array_equal(run("softmax", inp, "ordered_tree").view(np.uint32), first.view(np.uint32))


def test_ordered_tree_softmax_tiny_exponentials():
    """Outputs e / s are rounded once under every plan.  TREE plans compute
    them as q = e y, then q + (e - s q) y rounded once, y = 1 / s, and switch
    a wave to the division when one of its e lies in (0, 2^-96), where that
    form can be one unit off; ORDERED plans divide.  Rows here put x - max
    down to -104, so e runs through 2^-96 and the subnormals: whole rows of
    waves on the division, rows with one such e (one wave switches, the rest
    do not), and rows with none.  Every plan must give the same bits."""
    facts = lr.lr_device_facts_query()
    for rows, cols in [(9, 6144), (6, 1000), (4, 12288)]:
        rng = np.random.default_rng(rows * cols)
        x = np.empty((rows, cols), dtype=np.float32)
        for r in range(rows):
            kind = r % 3
            if kind == 0:    # spread to -104: most waves meet e < 2^-96
                x[r] = (-104.0 * rng.random(cols)).astype(np.float32)
            elif kind == 1:  # one element at -80 in an ordinary row
                x[r] = (-8.0 * rng.random(cols)).astype(np.float32)
                x[r, rng.integers(cols)] = -80.0
            else:            # none below 2^-96
                x[r] = (-30.0 * rng.random(cols)).astype(np.float32)
            x[r, rng.integers(cols)] = 0.0
        inp = {"x": x}
        plans = lr.lr_plan_enumerate(facts, "softmax", rows, cols, "ordered_tree", 1 if cols % 4 == 0 else 0)
        fams = sorted({p.family for p in plans})
        assert lr.LR_FAMILY_TREE in fams and lr.LR_FAMILY_ORDERED in fams, fams
        print(f"\n[gpu] softmax tiny exponentials {rows}x{cols}: {len(plans)} plans", flush=True)
        first = None
        for p in plans:
            got = run("softmax", inp, "ordered_tree", plan=p)
            check("softmax", inp, "ordered_tree", got, f"tiny exponentials {rows}x{cols} {p}")
            if first is None:
                first = got
            assert np.array_equal(got.view(np.uint32), first.view(np.uint32)), p
        sub = (first > 0) & (first < np.float32(2.0 ** -96))
        assert sub.any()  # the slow path's outputs are really there
