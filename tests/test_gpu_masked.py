"""Softmax and cross-entropy rows with masked (-infinity) elements, under
every legal plan of every policy.

Masked positions hold -inf, as an attention or vocabulary mask writes them;
each row keeps at least one finite element, the contract include/lr.h
states.  exp(-inf - max) = 0, so a masked element's softmax output is +0 and
it adds nothing to the sum of exponentials ("TIRx Metal reduction lowering",
section 1: softmax and cross-entropy are max, sum of exp(x - max) and the
division or logarithm).  The masks put whole waves' stripes at -inf (leading
and trailing runs, all but one element), which is where a wave's own maximum
is -inf.  Outputs are checked against the double oracle, and every masked
output must be exactly +0."""
import numpy as np
import pytest

import oracle
import row_reductions_amd as lr
import synth
from gpu_util import ATOL, RTOL, gamma_n, run_gpu

pytestmark = pytest.mark.gpu

POLICIES = ["unordered_tree", "ordered_fold", "ordered_tree", "fold_right"]
# aligned and misaligned rows, whole-wave and sub-wave teams, the headline
# shape, a row long enough for the STREAM family
SHAPES = [(8, 4096), (9, 1030), (6, 64), (5, 37), (3, 20000), (768, 6144)]


def masked_logits(rows, cols, seed):
    x = synth.normal_f32(seed, 0, rows * cols, 0.0, 4.0).reshape(rows, cols)
    rng = np.random.default_rng(seed)
    for r in range(rows):
        kind = r % 5
        if kind == 0:    # leading run: only the last 3% finite
            x[r, : cols - max(1, cols * 3 // 100)] = -np.inf
        elif kind == 1:  # trailing run (causal): only the first 100 finite
            x[r, min(cols - 1, 100):] = -np.inf
        elif kind == 2:  # all but one element, in the middle
            keep = cols // 2
            x[r, :] = -np.inf
            x[r, keep] = 1.5
        elif kind == 3:  # 90% masked at random, at least one kept
            m = rng.random(cols) < 0.9
            m[rng.integers(cols)] = False
            x[r, m] = -np.inf
        # kind 4: no mask
    return x


def check(op, x, got, ref, policy, what):
    cols = x.shape[1]
    g = 0.0 if policy == "unordered_tree" else gamma_n(cols - 1)
    err = np.abs(got.astype(np.float64) - ref)
    bound = ATOL + (RTOL + g) * np.abs(ref) + (g if op == "cross_entropy" else 0.0)
    if not (err <= bound).all():
        i = np.unravel_index(np.argmax(err - bound), ref.shape)
        raise AssertionError(f"{what}: at {i}: gpu={got[i]!r} ref={ref[i]!r}")


@pytest.mark.parametrize("op", ["softmax", "cross_entropy"])
def test_masked_rows_every_plan(op):
    facts = lr.lr_device_facts_query()
    n = 0
    for rows, cols in SHAPES:
        x = masked_logits(rows, cols, seed=rows * 7 + cols)
        if op == "softmax":
            inp = {"x": x}
            ref = oracle.softmax(x)
        else:
            # labels on finite logits, and one past the end (guard: fill 0)
            rng = np.random.default_rng(cols)
            lab = np.array([rng.choice(np.flatnonzero(np.isfinite(x[r]))) for r in range(rows)], dtype=np.int64)
            lab[0] = cols
            inp = {"logits": x, "labels": lab}
            ref = oracle.cross_entropy(x, lab)
        assert np.isfinite(ref).all()
        for policy in POLICIES:
            plans = lr.lr_plan_enumerate(facts, op, rows, cols, policy, 1 if cols % 4 == 0 else 0)
            if rows * cols > 100000:
                plans = plans[:: max(1, len(plans) // 12)] + [None]  # a sample and the automatic plan
            print(f"\n[gpu] masked {op} {rows}x{cols} {policy}: {len(plans)} plans", flush=True)
            for p in plans:
                got, st, _ = run_gpu(op, inp, None, policy, plan=p)
                assert st == lr.LR_OK, (p, lr.lr_status_string(st))
                what = f"{op} {rows}x{cols} {policy} {p}"
                check(op, x, got, ref, policy, what)
                if op == "softmax":
                    masked = np.isneginf(x)
                    assert (got[masked].view(np.uint32) == 0).all(), what  # +0 exactly
                n += 1
    assert n > 100


def test_ordered_softmax_of_tied_maxima_is_exact():
    """A row holding k copies of its maximum and -inf elsewhere has
    numerators exactly 1 and 0 (exp(0) = 1, exp(-inf) = 0) and sum exactly k
    (k < 2^24), so under an ordered policy, whose outputs are the quotient
    rounded once, each output is exactly fl(1/k) or +0: bit for bit, under
    every plan, whatever the device's exp does elsewhere."""
    facts = lr.lr_device_facts_query()
    for rows, cols in [(7, 4096), (5, 1030), (9, 64), (3, 20000)]:
        rng = np.random.default_rng(cols)
        x = np.full((rows, cols), -np.inf, dtype=np.float32)
        ks = []
        for r in range(rows):
            k = int(rng.integers(1, cols + 1)) if r % 2 else [1, 3, 7, 41, cols][r // 2 % 5]
            k = min(k, cols)
            x[r, rng.choice(cols, size=k, replace=False)] = 2.5
            ks.append(k)
        want = np.where(np.isneginf(x), np.float32(0.0),
                        (np.float32(1.0) / np.array(ks, dtype=np.float32))[:, None]).astype(np.float32)
        for policy in ["ordered_fold", "ordered_tree", "fold_right"]:
            plans = lr.lr_plan_enumerate(facts, "softmax", rows, cols, policy, 1 if cols % 4 == 0 else 0)
            print(f"\n[gpu] tied maxima {rows}x{cols} {policy}: {len(plans)} plans", flush=True)
            for p in plans + [None]:
                got, st, _ = run_gpu("softmax", {"x": x}, None, policy, plan=p)
                assert st == lr.LR_OK, (p, lr.lr_status_string(st))
                assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (rows, cols, policy, p)
