"""Pins of the CPU oracle to things other than itself.

Each check is a closed form, an invariant, a library routine the operation
reduces to, brute force on tiny rows with correctly rounded sums (math.fsum),
or a hand-worked golden value (tests/golden/worked_examples.json).  They are
chosen so that a dropped term, a wrong sign, a wrong index or stride, a
misplaced eps or a wrong fold order in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _rand(rows, cols, seed=7, mean=0.0, std=1.0):
    return synth.normal_f32(seed, 0, rows * cols, mean, std).reshape(rows, cols)


# --------------------------------------------------------------------------
# golden worked examples
# --------------------------------------------------------------------------

def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["op"])
def test_golden_worked_examples(case):
    op = case["op"]
    x = np.array(case["x"], dtype=np.float32)
    if op == "softmax":
        got = oracle.softmax(x)
    elif op == "rmsnorm":
        got = oracle.rmsnorm(x, case.get("gamma"), case["eps"])
    elif op == "layernorm":
        got = oracle.layernorm(x, case.get("gamma"), case.get("beta"), case["eps"])
    else:
        got = oracle.cross_entropy(x, np.array(case["labels"], dtype=np.int64))
    np.testing.assert_allclose(got, np.array(case["expected"]), rtol=1e-14, atol=1e-15)


# --------------------------------------------------------------------------
# softmax
# --------------------------------------------------------------------------

def test_softmax_rows_sum_to_one():
    for std in (0.1, 1.0, 4.0, 20.0):
        y = oracle.softmax(_rand(9, 1537, std=std))
        np.testing.assert_allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-13)
        assert (y >= 0).all()


def test_softmax_shift_invariance_dyadic_exact():
    # x = k/64 with |k| <= 2^10 and an integer shift c <= 2^10: x + c and x - max
    # are exact in float32 and in double, so the outputs must be bit-identical.
    rng = np.random.default_rng(1)
    k = rng.integers(-1024, 1025, size=(5, 300))
    x = (k / 64.0).astype(np.float32)
    for c in (1, 17, 1024, -513):
        assert np.array_equal(oracle.softmax(x + np.float32(c)), oracle.softmax(x))


def test_softmax_constant_row_and_two_element_closed_form():
    for n in (1, 2, 3, 7, 1537):
        y = oracle.softmax(np.full((2, n), 3.25, dtype=np.float32))
        assert np.array_equal(y, np.full((2, n), 1.0 / n))
    a = np.array([[0.5, -1.25], [3.0, 3.0], [-7.0, 2.0]], dtype=np.float32)
    y = oracle.softmax(a)
    for r in range(a.shape[0]):
        y0 = 1.0 / (1.0 + math.exp(float(a[r, 1]) - float(a[r, 0])))
        assert y[r, 0] == pytest.approx(y0, rel=1e-15)
        assert y[r, 1] == pytest.approx(1.0 - y0, rel=1e-14)


def test_softmax_large_offset_is_stable():
    # without the max subtraction exp(1000) overflows; with it the result is
    # independent of the offset.
    x = _rand(3, 257)
    y = oracle.softmax(x + np.float32(1000.0))
    assert np.isfinite(y).all()
    np.testing.assert_allclose(y, oracle.softmax(x.astype(np.float64) + 1000.0), rtol=1e-13)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, atol=1e-13)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 63, 64, 65, 127, 257])
def test_softmax_brute_force_tiny(n):
    x = _rand(3, n, seed=n, std=3.0)
    y = oracle.softmax(x)
    for r in range(3):
        row = [float(v) for v in x[r]]
        m = max(row)
        e = [math.exp(v - m) for v in row]
        s = math.fsum(e)
        for j in range(n):
            assert y[r, j] == pytest.approx(e[j] / s, rel=1e-13, abs=1e-300)
    # monotone in the input
    assert (np.argsort(x, axis=1, kind="stable") == np.argsort(y, axis=1, kind="stable")).all()


# --------------------------------------------------------------------------
# RMSNorm
# --------------------------------------------------------------------------

def test_rmsnorm_constant_row_is_gamma_sign():
    g = synth.uniform_f32(0, 1, 64, 0.5, 1.5)
    for c in (1.0, -1.0, 4.0, -0.125, 2.0 ** 20):
        x = np.full((2, 64), c, dtype=np.float32)
        y = oracle.rmsnorm(x, g, eps=0.0)
        assert np.array_equal(y, np.tile(g.astype(np.float64) * math.copysign(1.0, c), (2, 1)))
    # with eps > 0: gamma * c / sqrt(c^2 + eps)
    x = np.full((1, 10), 0.75, dtype=np.float32)
    eps = oracle.eps_as_f32(0.1)
    y = oracle.rmsnorm(x, g[:10], eps=0.1)
    np.testing.assert_allclose(y[0], g[:10].astype(np.float64) * 0.75 / math.sqrt(0.5625 + eps), rtol=1e-15)


def test_rmsnorm_scale_invariance_at_eps0_exact():
    x = _rand(4, 300)
    g = synth.uniform_f32(0, 1, 300, 0.5, 1.5)
    y = oracle.rmsnorm(x, g, eps=0.0)
    for k in (-6, 3, 10):
        assert np.array_equal(oracle.rmsnorm(x * np.float32(2.0 ** k), g, eps=0.0), y)


def test_rmsnorm_eps_placement():
    # mean_j (y_j / gamma_j)^2 = ms / (ms + eps): eps is added to the mean of
    # squares (not to the sum) inside the square root.
    x = _rand(6, 1000, std=0.5)
    g = synth.uniform_f32(0, 1, 1000, 0.5, 1.5)
    eps = 0.5
    y = oracle.rmsnorm(x, g, eps=eps)
    x64 = x.astype(np.float64)
    ms = np.mean(x64 * x64, axis=1)
    lhs = np.mean((y / g.astype(np.float64)) ** 2, axis=1)
    np.testing.assert_allclose(lhs, ms / (ms + eps), rtol=1e-13)


@pytest.mark.parametrize("n", [1, 2, 3, 5, 64, 65, 257])
def test_rmsnorm_brute_force_tiny(n):
    x = _rand(3, n, seed=100 + n)
    g = synth.uniform_f32(5, 1, n, 0.5, 1.5)
    eps = oracle.eps_as_f32(1e-6)
    y = oracle.rmsnorm(x, g, eps=1e-6)
    for r in range(3):
        row = [float(v) for v in x[r]]
        d = math.sqrt(math.fsum(v * v for v in row) / n + eps)
        for j in range(n):
            assert y[r, j] == pytest.approx(float(g[j]) * row[j] / d, rel=1e-14)
    # gamma omitted means gamma = 1
    np.testing.assert_array_equal(oracle.rmsnorm(x, None, 1e-6),
                                  oracle.rmsnorm(x, np.ones(n, np.float32), 1e-6))


# --------------------------------------------------------------------------
# LayerNorm
# --------------------------------------------------------------------------

def test_layernorm_mean_zero_variance_closed_form():
    x = _rand(5, 1537, mean=3.0, std=2.0)
    x64 = x.astype(np.float64)
    v = np.var(x64, axis=1)
    for eps in (0.0, 1e-5, 0.3):
        e = oracle.eps_as_f32(eps)
        y = oracle.layernorm(x, None, None, eps)
        np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
        np.testing.assert_allclose(np.var(y, axis=1), v / (v + e), rtol=1e-12)


def test_layernorm_reduces_to_numpy_standardisation():
    x = _rand(4, 12289, mean=3.0, std=2.0)
    x64 = x.astype(np.float64)
    eps = oracle.eps_as_f32(1e-5)
    ref = (x64 - x64.mean(axis=1, keepdims=True)) / np.sqrt(x64.var(axis=1, keepdims=True) + eps)
    np.testing.assert_allclose(oracle.layernorm(x, None, None, 1e-5), ref, rtol=1e-11, atol=1e-12)


def test_layernorm_centred_variance_at_large_mean():
    # mean 2^20, std 4: the uncentred E[x^2] - E[x]^2 loses ~1e-4 of the
    # variance in double; the centred two-pass keeps it to ~1e-13.
    x = _rand(3, 4096, mean=2.0 ** 20, std=4.0)
    mu, var = oracle.layernorm_stats(x)
    x64 = x.astype(np.float64)
    np.testing.assert_allclose(mu, x64.mean(axis=1), rtol=1e-15)
    np.testing.assert_allclose(var, x64.var(axis=1), rtol=1e-10)


def test_layernorm_constant_row_is_beta_and_affine_relation():
    g = synth.uniform_f32(0, 1, 33, 0.5, 1.5)
    b = synth.normal_f32(0, 2, 33, 0.0, 0.1)
    x = np.full((3, 33), -2.5, dtype=np.float32)
    assert np.array_equal(oracle.layernorm(x, g, b, 1e-5), np.tile(b.astype(np.float64), (3, 1)))
    x = _rand(3, 33)
    y0 = oracle.layernorm(x, None, None, 1e-5)
    y = oracle.layernorm(x, g, b, 1e-5)
    np.testing.assert_allclose(y, y0 * g.astype(np.float64) + b.astype(np.float64), rtol=1e-14,
                               atol=1e-16)


def test_layernorm_shift_invariance_dyadic():
    rng = np.random.default_rng(3)
    x = (rng.integers(-1024, 1025, size=(4, 200)) / 64.0).astype(np.float32)
    y = oracle.layernorm(x, None, None, 1e-5)
    for c in (5, -300, 1024):
        np.testing.assert_allclose(oracle.layernorm(x + np.float32(c), None, None, 1e-5), y,
                                   rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("n", [1, 2, 3, 5, 64, 65, 257])
def test_layernorm_brute_force_tiny(n):
    x = _rand(3, n, seed=200 + n, mean=3.0, std=2.0)
    g = synth.uniform_f32(5, 1, n, 0.5, 1.5)
    b = synth.normal_f32(5, 2, n, 0.0, 0.1)
    eps = oracle.eps_as_f32(1e-5)
    y = oracle.layernorm(x, g, b, 1e-5)
    for r in range(3):
        row = [float(v) for v in x[r]]
        mu = math.fsum(row) / n
        var = math.fsum((v - mu) ** 2 for v in row) / n
        d = math.sqrt(var + eps)
        for j in range(n):
            assert y[r, j] == pytest.approx((row[j] - mu) / d * float(g[j]) + float(b[j]),
                                            rel=1e-12, abs=1e-13)


# --------------------------------------------------------------------------
# fused residual LayerNorm
# --------------------------------------------------------------------------

def _res_inputs(rows, cols, seed=11):
    d = synth.add_layernorm_inputs(rows, cols, seed=seed)
    return d["x"], d["residual"], d["gamma"], d["beta"]


def test_add_layernorm_zero_residual_is_layernorm():
    # x + 0.0f == x exactly, so the fused op must equal LayerNorm of x bit for bit
    x, _, g, b = _res_inputs(4, 1537)
    z = np.zeros_like(x)
    assert np.array_equal(oracle.add_layernorm(x, z, g, b, 1e-5), oracle.layernorm(x, g, b, 1e-5))


def test_add_layernorm_is_symmetric_in_its_inputs():
    x, r, g, b = _res_inputs(3, 1000)
    assert np.array_equal(oracle.add_layernorm(x, r, g, b, 1e-5), oracle.add_layernorm(r, x, g, b, 1e-5))


def test_add_layernorm_combined_is_float32_sum():
    # the combined tensor is one IEEE single-precision addition per element
    x, r, g, b = _res_inputs(3, 777)
    _, s = oracle.add_layernorm(x, r, g, b, 1e-5, with_sum=True)
    assert s.dtype == np.float32
    assert np.array_equal(s, np.add(x, r, dtype=np.float32))
    # and it differs from the exact (double) sum somewhere, so the FP32 rounding is observable
    assert not np.array_equal(s.astype(np.float64), x.astype(np.float64) + r.astype(np.float64))


def test_add_layernorm_reduces_to_numpy_standardisation_of_fp32_sum():
    x, r, g, b = _res_inputs(4, 6144)
    c = np.add(x, r, dtype=np.float32).astype(np.float64)
    eps = oracle.eps_as_f32(1e-5)
    ref = (c - c.mean(axis=1, keepdims=True)) / np.sqrt(c.var(axis=1, keepdims=True) + eps)
    ref = ref * g.astype(np.float64) + b.astype(np.float64)
    np.testing.assert_allclose(oracle.add_layernorm(x, r, g, b, 1e-5), ref, rtol=1e-11, atol=1e-12)
    # the double-precision sum is a different (rejected) reading: it moves outputs by ~1e-7
    exact = x.astype(np.float64) + r.astype(np.float64)
    ref2 = (exact - exact.mean(axis=1, keepdims=True)) / np.sqrt(exact.var(axis=1, keepdims=True) + eps)
    ref2 = ref2 * g.astype(np.float64) + b.astype(np.float64)
    assert np.abs(ref2 - ref).max() > 1e-9


def test_add_layernorm_constant_combination_is_beta():
    # dyadic x and c - x are exact in FP32, so every combined value is c: y = beta exactly
    rng = np.random.default_rng(5)
    x = (rng.integers(-1024, 1025, size=(3, 129)) / 64.0).astype(np.float32)
    r = (np.float32(7.5) - x).astype(np.float32)
    g = synth.uniform_f32(0, 1, 129, 0.5, 1.5)
    b = synth.normal_f32(0, 2, 129, 0.0, 0.1)
    assert np.array_equal(oracle.add_layernorm(x, r, g, b, 1e-5), np.tile(b.astype(np.float64), (3, 1)))


def test_add_layernorm_mean_zero_variance_closed_form():
    x, r, _, _ = _res_inputs(3, 2049)
    c = np.add(x, r, dtype=np.float32).astype(np.float64)
    v = np.var(c, axis=1)
    e = oracle.eps_as_f32(1e-5)
    y = oracle.add_layernorm(x, r, None, None, 1e-5)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose(np.var(y, axis=1), v / (v + e), rtol=1e-12)


@pytest.mark.parametrize("n", [1, 2, 5, 64, 257])
def test_add_layernorm_brute_force_tiny(n):
    x, r, g, b = _res_inputs(2, n, seed=300 + n)
    eps = oracle.eps_as_f32(1e-5)
    y = oracle.add_layernorm(x, r, g, b, 1e-5)
    for i in range(2):
        row = [float(np.float32(x[i, j]) + np.float32(r[i, j])) for j in range(n)]
        mu = math.fsum(row) / n
        var = math.fsum((v - mu) ** 2 for v in row) / n
        d = math.sqrt(var + eps)
        for j in range(n):
            assert y[i, j] == pytest.approx((row[j] - mu) / d * float(g[j]) + float(b[j]),
                                            rel=1e-12, abs=1e-13)


# --------------------------------------------------------------------------
# row sum, row minimum and maximum
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 3, 127, 257, 1024])
def test_row_sum_brute_force_fsum(n):
    x = _rand(4, n, seed=400 + n, mean=0.5, std=3.0)
    got = oracle.row_sum(x)
    for r in range(4):
        row = [float(v) for v in x[r]]
        exact = math.fsum(row)
        # double accumulation of n terms: within n * 2^-53 * sum |x| of the exact sum
        assert abs(got[r] - exact) <= n * 2.0 ** -53 * math.fsum(abs(v) for v in row) + 1e-300


def test_row_sum_exact_cases():
    # integers and dyadic values: every partial sum is exact
    rng = np.random.default_rng(8)
    k = rng.integers(-4096, 4097, size=(5, 4096))
    x = (k / 8.0).astype(np.float32)
    assert np.array_equal(oracle.row_sum(x), k.sum(axis=1) / 8.0)
    assert np.array_equal(oracle.row_sum(np.ones((3, 257), np.float32)), np.full(3, 257.0))
    # rows are independent and use stride cols
    x = _rand(6, 129)
    assert np.array_equal(oracle.row_sum(x)[2:5], oracle.row_sum(x[2:5]))


def test_row_sum_matches_numpy_pairwise():
    x = _rand(7, 4096, std=2.0)
    np.testing.assert_allclose(oracle.row_sum(x), x.astype(np.float64).sum(axis=1), rtol=0, atol=1e-11)


@pytest.mark.parametrize("n", [1, 2, 5, 1024, 4097])
def test_row_minmax_matches_numpy_and_is_order_free(n):
    x = _rand(7, n, seed=500 + n, std=5.0)
    lo, hi = oracle.row_minmax(x)
    assert np.array_equal(lo, x.min(axis=1)) and np.array_equal(hi, x.max(axis=1))
    perm = np.random.default_rng(n).permutation(n)
    lo2, hi2 = oracle.row_minmax(x[:, perm])
    assert np.array_equal(lo, lo2) and np.array_equal(hi, hi2)
    assert (lo <= hi).all()


def test_row_minmax_extremes_at_the_ends():
    # the extremes sit in the first and the last column: a loop that skips
    # either end fails
    x = np.zeros((3, 50), np.float32)
    x[:, 0] = -7.0
    x[:, -1] = 9.0
    x[1, 0], x[1, -1] = 9.5, -8.0
    lo, hi = oracle.row_minmax(x)
    assert list(lo) == [-7.0, -8.0, -7.0] and list(hi) == [9.0, 9.5, 9.0]


# --------------------------------------------------------------------------
# cross-entropy
# --------------------------------------------------------------------------

def test_cross_entropy_is_logsumexp_minus_selected():
    x = _rand(16, 4096, std=2.0)
    lab = synth.labels_i64(0, 3, 16, 0, 4096)
    ref = logsumexp(x.astype(np.float64), axis=1) - x[np.arange(16), lab].astype(np.float64)
    np.testing.assert_allclose(oracle.cross_entropy(x, lab), ref, rtol=1e-13)


def test_cross_entropy_guard_out_of_range_is_logsumexp():
    x = _rand(7, 300, std=2.0)
    lse = logsumexp(x.astype(np.float64), axis=1)
    bad = np.array([-1, 300, 2 ** 31, 2 ** 32 + 3, -(2 ** 63), 2 ** 63 - 1, 2 ** 32 + 5],
                   dtype=np.int64)
    np.testing.assert_allclose(oracle.cross_entropy(x, bad), lse, rtol=1e-14)
    # labels whose low 32 bits are in range but whose high bits are not must
    # still fail the guard (int64 compare)
    alias = np.array([2 ** 32 + 5] * 7, dtype=np.int64)
    np.testing.assert_allclose(oracle.cross_entropy(x, alias), lse, rtol=1e-14)


def test_cross_entropy_closed_forms():
    for n in (1, 2, 10, 32000):
        x = np.full((1, n), 0.75, dtype=np.float32)
        assert oracle.cross_entropy(x, np.array([n - 1]))[0] == pytest.approx(math.log(n), rel=1e-14,
                                                                              abs=1e-15)
    # two classes: loss = softplus(x_other - x_label)
    a = np.array([[0.5, -1.25], [3.0, 9.0]], dtype=np.float32)
    got = oracle.cross_entropy(a, np.array([0, 0]))
    for r in range(2):
        d = float(a[r, 1]) - float(a[r, 0])
        assert got[r] == pytest.approx(math.log1p(math.exp(d)), rel=1e-14)


def test_cross_entropy_matches_minus_log_softmax():
    x = _rand(5, 777, std=2.0)
    lab = synth.labels_i64(1, 3, 5, 0, 777)
    p = oracle.softmax(x)
    np.testing.assert_allclose(oracle.cross_entropy(x, lab), -np.log(p[np.arange(5), lab]),
                               rtol=1e-12)


def test_cross_entropy_ramp_makes_index_errors_exact():
    n = 4096
    x = np.tile((np.arange(n) * 2.0 ** -8).astype(np.float32), (8, 1))
    lab = np.array([0, 1, 2, 100, 2047, 4094, 4095, 17], dtype=np.int64)
    loss = oracle.cross_entropy(x, lab)
    lse = logsumexp(x[0].astype(np.float64))
    np.testing.assert_allclose(loss, lse - lab * 2.0 ** -8, rtol=0, atol=1e-12)


def test_cross_entropy_large_offset_is_stable():
    # dyadic logits k/64 so that x + 1000 is exact in float32; without the max
    # shift exp(1000) overflows
    rng = np.random.default_rng(5)
    x = (rng.integers(-512, 513, size=(3, 500)) / 64.0).astype(np.float32)
    lab = np.array([1, 2, 3])
    a = oracle.cross_entropy(x + np.float32(1000.0), lab)
    assert np.isfinite(a).all()
    np.testing.assert_allclose(a, oracle.cross_entropy(x, lab), rtol=1e-13)


# --------------------------------------------------------------------------
# FP32 ordered-fold replay
# --------------------------------------------------------------------------

def test_fold_left_order_is_left_to_right():
    big = 2.0 ** 24
    # 2^24 + 1 rounds back to 2^24 (tie to even), so the left fold absorbs each 1
    assert oracle.fold_left_f32([big, 1, 1, 1, 1], 0) == big
    # ones first: 4 + 2^24 is exact
    assert oracle.fold_left_f32([1, 1, 1, 1, big], 0) == big + 4
    # a double accumulator would give 2^24 + 4 in the first case too


def test_fold_left_rounds_square_and_add_separately():
    # c0 = (2^-12)^2 = 2^-24; x1^2 = 1 + 2^-11 + 2^-24 rounds (tie to even) to
    # 1 + 2^-11; then 2^-24 + (1 + 2^-11) ties back to 1 + 2^-11.  A fused
    # multiply-add (or a double accumulator) gives 1 + 2^-11 + 2^-23 instead.
    x = [2.0 ** -12, 1.0 + 2.0 ** -12]
    got = oracle.fold_left_f32(x, 1)
    assert got == 1.0 + 2.0 ** -11
    assert got != 1.0 + 2.0 ** -11 + 2.0 ** -23


def test_fold_replay_constant_rows():
    g = synth.uniform_f32(0, 1, 48, 0.5, 1.5)
    b = synth.normal_f32(0, 2, 48, 0.0, 0.1)
    x = np.full((2, 48), 2.0 ** 3, dtype=np.float32)
    # ms = 64 exactly, r = 1/8, x*r = 1, so y = gamma bit for bit
    assert np.array_equal(oracle.rmsnorm_fold_f32(x, g, 0.0), np.tile(g, (2, 1)))
    x = np.full((2, 48), -1.75, dtype=np.float32)
    assert np.array_equal(oracle.layernorm_fold_f32(x, g, b, 1e-5), np.tile(b, (2, 1)))


@pytest.mark.parametrize("op", ["rmsnorm", "layernorm"])
def test_fold_replay_within_serial_error_of_double_oracle(op):
    # 256 x 3072 RMSNorm (x ~ N(0,1)) and a LayerNorm row set; the serial FP32
    # sum of n terms errs by at most about n * 2^-24 relative, far inside the
    # 1e-6 + 1e-5 |ref| parity bar.
    if op == "rmsnorm":
        inp = synth.rmsnorm_inputs(64, 3072, seed=0)
        ref = oracle.rmsnorm(inp["x"], inp["gamma"], 1e-6)
        got = oracle.rmsnorm_fold_f32(inp["x"], inp["gamma"], 1e-6)
    else:
        inp = synth.layernorm_inputs(16, 6144, seed=0)
        ref = oracle.layernorm(inp["x"], inp["gamma"], inp["beta"], 1e-5)
        got = oracle.layernorm_fold_f32(inp["x"], inp["gamma"], inp["beta"], 1e-5)
    err = np.abs(got.astype(np.float64) - ref)
    assert (err <= 1e-6 + 1e-5 * np.abs(ref)).all()
    assert err.max() > 0  # the replay really is FP32


ORDERED = ["ordered_fold", "ordered_tree", "fold_right"]
GOLDEN_ORDERED = os.path.join(os.path.dirname(__file__), "golden", "ordered_sums.json")


def _ordered_cases():
    with open(GOLDEN_ORDERED) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _ordered_cases(), ids=lambda c: str(c["x"]))
def test_ordered_sums_golden(case):
    x = np.array(case["x"], dtype=np.float32)
    for pol, key in (("ordered_fold", "fold_left"), ("ordered_tree", "ordered_tree"), ("fold_right", "fold_right")):
        assert oracle.ordered_sum_f32(x, pol, case["kind"]) == case[key], (pol, case)


def test_fold_right_is_fold_left_of_the_reversed_row():
    for n in (1, 2, 7, 1000, 4097):
        x = _rand(1, n, seed=600 + n, mean=1.0, std=5.0)[0]
        for kind in (0, 1):
            a = oracle.ordered_sum_f32(x, "fold_right", kind)
            b = oracle.ordered_sum_f32(x[::-1].copy(), "ordered_fold", kind)
            assert np.float32(a).view(np.uint32) == np.float32(b).view(np.uint32)


def test_tree_zero_padding_and_halves():
    rng = np.random.default_rng(12)
    for n in (1, 3, 5, 100, 257, 1000):
        x = rng.normal(size=n).astype(np.float32)
        p = 1
        while p < n:
            p *= 2
        # padding with -0 (the add identity) up to the tree's own width, or
        # beyond, changes nothing
        for extra in (p - n, 2 * p - n, 4 * p - n):
            xp = np.concatenate([x, np.full(extra, -0.0, np.float32)])
            assert oracle.ordered_sum_f32(xp, "ordered_tree") == oracle.ordered_sum_f32(x, "ordered_tree")
    # a full tree is the rounded sum of its two half trees
    for k in range(1, 12):
        x = rng.normal(size=2 ** k).astype(np.float32)
        h = 2 ** (k - 1)
        whole = oracle.ordered_sum_f32(x, "ordered_tree")
        halves = np.float32(np.float32(oracle.ordered_sum_f32(x[:h], "ordered_tree")) +
                            np.float32(oracle.ordered_sum_f32(x[h:], "ordered_tree")))
        assert np.float32(whole) == halves


def test_tree_of_negative_zeros_is_negative_zero():
    """IEEE 754 (section 6.3): a sum of negative zeros is -0, and -0 is the
    exact add identity (x + -0 == x, sign included).  A tree padded with +0
    instead would turn a row of negative zeros into +0 whenever it pads; so
    would padding a power-of-two row any further."""
    for n in (1, 2, 3, 4, 5, 64, 100, 256, 257):
        x = np.full(n, -0.0, np.float32)
        t = np.float32(oracle.ordered_sum_f32(x, "ordered_tree"))
        assert t == 0.0 and math.copysign(1.0, t) == -1.0, n
        # one +0 anywhere makes the exact sum +0
        x[n // 2] = 0.0
        t = np.float32(oracle.ordered_sum_f32(x, "ordered_tree"))
        assert t == 0.0 and math.copysign(1.0, t) == 1.0, n
    # the padding keeps every value's sign and bits, zeros included
    for v in (-0.0, 0.0, -1.5, 3.0e-45):
        x = np.array([v, -0.0, -0.0], np.float32)
        assert np.float32(oracle.ordered_sum_f32(x, "ordered_tree")).view(np.uint32) == np.float32(v).view(np.uint32)


def test_tree_leaf_pairs_commute_but_left_fold_does_not():
    rng = np.random.default_rng(13)
    # magnitudes spread over twelve decades, so that every reordering is visible in a serial chain
    x = (rng.normal(size=4096) * 10.0 ** rng.uniform(-4, 8, size=4096)).astype(np.float32)
    sw = x.reshape(-1, 2)[:, ::-1].reshape(-1).copy()
    assert oracle.ordered_sum_f32(sw, "ordered_tree") == oracle.ordered_sum_f32(x, "ordered_tree")
    assert oracle.ordered_sum_f32(sw, "ordered_fold") != oracle.ordered_sum_f32(x, "ordered_fold")


@pytest.mark.parametrize("pol", ORDERED)
def test_ordered_sums_exact_on_integers_and_within_bound(pol):
    rng = np.random.default_rng(14)
    k = rng.integers(-1000, 1001, size=5000)
    assert oracle.ordered_sum_f32(k.astype(np.float32), pol) == float(k.sum())
    for n in (3, 1000, 65536):
        x = rng.normal(size=n).astype(np.float32)
        exact = math.fsum(float(v) for v in x)
        steps = math.ceil(math.log2(n)) if pol == "ordered_tree" else n - 1
        g = steps * 2.0 ** -24 / (1 - steps * 2.0 ** -24)
        assert abs(oracle.ordered_sum_f32(x, pol) - exact) <= g * float(np.abs(x.astype(np.float64)).sum())


@pytest.mark.parametrize("pol", ORDERED)
def test_ordered_norm_replays(pol):
    x = _rand(5, 1537, mean=3.0, std=2.0)
    g = synth.uniform_f32(0, 1, 1537, 0.5, 1.5)
    b = synth.normal_f32(0, 2, 1537, 0.0, 0.1)
    # fold_left replays agree with the earlier (pinned) fold replays bit for bit
    if pol == "ordered_fold":
        assert np.array_equal(oracle.rmsnorm_ordered_f32(x, g, 1e-6, pol), oracle.rmsnorm_fold_f32(x, g, 1e-6))
        assert np.array_equal(oracle.layernorm_ordered_f32(x, g, b, 1e-5, pol), oracle.layernorm_fold_f32(x, g, b, 1e-5))
    # every replay is within FP32 rounding of the double definition
    np.testing.assert_allclose(oracle.rmsnorm_ordered_f32(x, g, 1e-6, pol), oracle.rmsnorm(x, g, 1e-6), rtol=2e-5, atol=1e-6)
    np.testing.assert_allclose(oracle.layernorm_ordered_f32(x, g, b, 1e-5, pol), oracle.layernorm(x, g, b, 1e-5),
                               rtol=5e-4, atol=5e-5)
    # constant rows: RMSNorm gives gamma*sign exactly at eps = 0 (c = 2^k), LayerNorm gives beta
    c = np.full((2, 1537), -4.0, np.float32)
    assert np.array_equal(oracle.rmsnorm_ordered_f32(c, g, 0.0, pol), np.tile(-g, (2, 1)))
    assert np.array_equal(oracle.layernorm_ordered_f32(c, g, b, 1e-5, pol), np.tile(b, (2, 1)))
    # the three policies generally disagree in the last bits (the order is observable)
    if pol != "ordered_fold":
        y = oracle.layernorm_ordered_f32(x, g, b, 1e-5, pol)
        assert not np.array_equal(y, oracle.layernorm_ordered_f32(x, g, b, 1e-5, "ordered_fold"))


def test_fold_replay_rows_are_independent():
    inp = synth.layernorm_inputs(5, 300, seed=4)
    full = oracle.layernorm_fold_f32(inp["x"], inp["gamma"], inp["beta"], 1e-5)
    for r in range(5):
        one = oracle.layernorm_fold_f32(inp["x"][r:r + 1], inp["gamma"], inp["beta"], 1e-5)
        assert np.array_equal(one[0], full[r])


# --------------------------------------------------------------------------
# the ordered replays' FP32 steps after the fold, against hand-worked values
# (tests/golden/ordered_post_fold.json: the mean as acc / cols, IEEE division
# and square root, (x * r) * gamma, ((x - mu) * r) * gamma + beta, each
# rounded on its own; "TIRx Metal reduction lowering", section 1)
# --------------------------------------------------------------------------

GOLDEN_POST_FOLD = os.path.join(os.path.dirname(__file__), "golden", "ordered_post_fold.json")


def _post_fold_cases():
    with open(GOLDEN_POST_FOLD) as f:
        return json.load(f)["cases"]


def _post_fold_replays(case):
    """Every FP32 replay of the case's operation: the fold_left replay and the
    replays under each ordered policy (the rows' sums are exact integers, so
    the order cannot change them)."""
    x = np.array([case["x"]], dtype=np.float32)
    g = None if case.get("gamma") is None else np.array(case["gamma"], dtype=np.float32)
    eps = case["eps"]
    if case["op"] == "rmsnorm":
        yield "fold_f32", oracle.rmsnorm_fold_f32(x, g, eps)
        for pol in ORDERED:
            yield pol, oracle.rmsnorm_ordered_f32(x, g, eps, pol)
    else:
        b = None if case.get("beta") is None else np.array(case["beta"], dtype=np.float32)
        yield "fold_f32", oracle.layernorm_fold_f32(x, g, b, eps)
        for pol in ORDERED:
            yield pol, oracle.layernorm_ordered_f32(x, g, b, eps, pol)


@pytest.mark.parametrize("case", _post_fold_cases(), ids=lambda c: c["name"])
def test_ordered_post_fold_golden(case):
    want = np.array(case["expected"], dtype=np.float32).view(np.uint32)
    for name, y in _post_fold_replays(case):
        got = y[0].view(np.uint32)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (name, case["name"], bad[:4], y[0][bad[:4]])


def test_ordered_post_fold_golden_values_are_the_stated_mantissas():
    """The decimal values in the golden file are the m * 2^e forms its
    derivations give (read here as exact binary fractions, not recomputed)."""
    cases = {c["name"]: c for c in _post_fold_cases()}
    ln = np.array(cases["layernorm_scale_gamma_beta_each_rounded"]["expected"], dtype=np.float32)
    assert float(ln[0]) == 97867104 * 2.0 ** -25
    assert float(ln[1]) == -78293680 * 2.0 ** -25
    assert float(ln[2]) == 0.0
    assert all(abs(float(v)) == 11184811 * 2.0 ** -25 for v in ln[3:])
    rms = cases["rmsnorm_scales_then_applies_gamma"]
    assert rms["expected"] == rms["gamma"]
