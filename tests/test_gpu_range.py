"""FP32 range at the small end of the norms' inputs and the large end of the
logits, under every legal plan of every policy.

RMSNorm and LayerNorm with eps = 0 on rows x = 2^-64 z, z ~ N(0, 1): every
square (x^2 ~ 2^-128 z^2) and the mean square or variance are FP32
subnormals, so the reciprocal square root of the row statistic takes an
argument below 2^-126 ("TIRx Metal reduction lowering", section 1: the norms
are a sum of squares, its mean and its inverse root; section 5.1 for
LayerNorm's centred form).  The squares still carry 21 bits, so the
unordered outputs stay within |gpu - ref| <= 1e-6 + 1e-5 |ref| of the double
oracle, and the ordered policies, whose every operation is IEEE, equal the
FP32 replays bit for bit; at 2^-72 (squares with a handful of bits, some
flushed to zero by rounding) the ordered results must still equal the
replays.  Softmax and cross-entropy on logits of spread 1000, where every
exponential but the maximum's underflows, stay within the bar."""
import numpy as np
import pytest
import torch

import oracle
import row_reductions_amd as lr
import synth
from gpu_util import ATOL, DEV, RTOL, assert_parity, bits_equal, gamma_n, run_gpu

pytestmark = pytest.mark.gpu

POLICIES = ["unordered_tree", "ordered_fold", "ordered_tree", "fold_right"]
# whole-wave and sub-wave teams, a ragged width, a row for the STREAM family,
# the LayerNorm workload's width
SHAPES = [(6, 1024), (5, 37), (3, 6144), (4, 20000), (2, 12289)]


def tiny_rows(rows, cols, seed, log2_scale):
    z = synth.normal_f32(seed, 0, rows * cols, 0.0, 1.0).reshape(rows, cols)
    return (z * np.float32(2.0 ** log2_scale)).astype(np.float32)  # exact: a power of two


def params(op, cols, seed):
    rng = np.random.default_rng(seed)
    g = (rng.random(cols) + 0.5).astype(np.float32)
    b = (rng.standard_normal(cols) * 0.1).astype(np.float32)
    return {"gamma": g} if op == "rmsnorm" else {"gamma": g, "beta": b}


def replay(op, inp, policy):
    if op == "rmsnorm":
        return oracle.rmsnorm_ordered_f32(inp["x"], inp.get("gamma"), 0.0, policy)
    return oracle.layernorm_ordered_f32(inp["x"], inp.get("gamma"), inp.get("beta"), 0.0, policy)


def plans_of(facts, op, rows, cols, policy):
    plans = lr.lr_plan_enumerate(facts, op, rows, cols, policy, 1 if cols % 4 == 0 else 0)
    if len(plans) > 40:
        plans = plans[:: len(plans) // 40 + 1]
    return plans + [None]


@pytest.mark.parametrize("op", ["rmsnorm", "layernorm"])
def test_subnormal_statistics_with_zero_eps(op):
    facts = lr.lr_device_facts_query()
    n = 0
    for k, (rows, cols) in enumerate(SHAPES):
        x = tiny_rows(rows, cols, seed=cols + k, log2_scale=-64)
        inp = {"x": x, **(params(op, cols, cols) if k % 2 else {})}
        sq = x.astype(np.float32) ** 2
        assert (sq < np.float32(2.0 ** -126)).mean() > 0.9  # the squares are subnormal
        ref = oracle.rmsnorm(x, inp.get("gamma"), 0.0) if op == "rmsnorm" else \
            oracle.layernorm(x, inp.get("gamma"), inp.get("beta"), 0.0)
        for policy in POLICIES:
            plans = plans_of(facts, op, rows, cols, policy)
            rep = None if policy == "unordered_tree" else replay(op, inp, policy)
            print(f"\n[gpu] subnormal {op} {rows}x{cols} {policy}: {len(plans)} plans", flush=True)
            for p in plans:
                got, st, _ = run_gpu(op, inp, 0.0, policy, plan=p)
                assert st == lr.LR_OK, (p, lr.lr_status_string(st))
                what = f"subnormal {op} {rows}x{cols} {policy} {p}"
                if rep is None:
                    assert_parity(got, ref, what)
                else:
                    bits_equal(got, rep, what)
                n += 1
    assert n > 300


@pytest.mark.parametrize("op", ["rmsnorm", "layernorm"])
def test_ordered_replays_hold_where_squares_lose_bits(op):
    facts = lr.lr_device_facts_query()
    for k, (rows, cols) in enumerate(SHAPES[:3]):
        x = tiny_rows(rows, cols, seed=7 * cols + k, log2_scale=-72)
        inp = {"x": x, **params(op, cols, cols + 1)}
        for policy in POLICIES[1:]:
            rep = replay(op, inp, policy)
            assert np.isfinite(rep).all()
            plans = plans_of(facts, op, rows, cols, policy)
            print(f"\n[gpu] 2^-72 {op} {rows}x{cols} {policy}: {len(plans)} plans", flush=True)
            for p in plans:
                got, st, _ = run_gpu(op, inp, 0.0, policy, plan=p)
                assert st == lr.LR_OK, (p, lr.lr_status_string(st))
                bits_equal(got, rep, f"2^-72 {op} {rows}x{cols} {policy} {p}")


def test_add_layernorm_subnormal_variance():
    """The fused residual LayerNorm: combined = fl32(x + residual) with both
    at 2^-64 scale, eps = 0, the automatic plan of every policy."""
    rows, cols = 8, 6144
    x = tiny_rows(rows, cols, 3, -64)
    r = tiny_rows(rows, cols, 4, -64)
    p = params("layernorm", cols, 5)
    c = (x + r).astype(np.float32)
    ref = oracle.add_layernorm(x, r, p["gamma"], p["beta"], 0.0)
    for policy in POLICIES:
        xv, rv = torch.from_numpy(x).to(DEV), torch.from_numpy(r).to(DEV)
        gv, bv = torch.from_numpy(p["gamma"]).to(DEV), torch.from_numpy(p["beta"]).to(DEV)
        y = torch.empty(rows, cols, dtype=torch.float32, device=DEV)
        st = lr.lr_add_layernorm_f32(xv, rv, gv, bv, y, None, rows, cols, 0.0, policy)
        assert st == lr.LR_OK, lr.lr_status_string(st)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        if policy == "unordered_tree":
            assert_parity(got, ref, "add_layernorm 2^-64")
        else:
            bits_equal(got, oracle.layernorm_ordered_f32(c, p["gamma"], p["beta"], 0.0, policy),
                       f"add_layernorm 2^-64 [{policy}]")


@pytest.mark.parametrize("op", ["softmax", "cross_entropy"])
def test_logits_of_large_spread(op):
    facts = lr.lr_device_facts_query()
    for rows, cols in [(4, 4096), (3, 1030), (2, 32000)]:
        x = synth.normal_f32(cols, 0, rows * cols, 0.0, 1000.0).reshape(rows, cols)
        if op == "softmax":
            inp, ref = {"x": x}, oracle.softmax(x)
        else:
            lab = np.random.default_rng(cols).integers(0, cols, rows).astype(np.int64)
            lab[0] = int(np.argmax(x[0]))  # a loss of exactly 0 next to losses near 1e3
            inp, ref = {"logits": x, "labels": lab}, oracle.cross_entropy(x, lab)
        for policy in POLICIES:
            g = 0.0 if policy == "unordered_tree" else gamma_n(cols - 1)
            plans = plans_of(facts, op, rows, cols, policy)
            print(f"\n[gpu] spread 1000 {op} {rows}x{cols} {policy}: {len(plans)} plans", flush=True)
            for p in plans:
                got, st, _ = run_gpu(op, inp, None, policy, plan=p)
                assert st == lr.LR_OK, (p, lr.lr_status_string(st))
                err = np.abs(got.astype(np.float64) - ref)
                bound = ATOL + (RTOL + g) * np.abs(ref) + (g if op == "cross_entropy" else 0.0)
                assert (err <= bound).all(), (op, rows, cols, policy, p, float((err / bound).max()))
