"""GPU parity: the HIP path through the C ABI against the CPU oracle, element
by element.

unordered_tree results must satisfy |gpu - ref| <= 1e-6 + 1e-5 |ref| against
the double oracle everywhere.  ordered_fold results must satisfy that bar on
the listed workloads, and everywhere else must equal the CPU FP32 left-fold
replay bit for bit (RMSNorm, LayerNorm) or stay within the bar widened by the
serial-sum bound (softmax, cross-entropy): a strict FP32 left fold over long
rows carries more rounding than 1e-5 allows (gpu_util.check_output).

Covers the five workloads at full size (both policies where they are
listed), a ragged sweep of widths and row counts, every legal plan forced
through the explicit-plan entry points, misaligned row starts, in-place
calls and untouched canary padding around the output."""
import numpy as np
import pytest

import oracle
import row_reductions_amd as lr
import synth
from gpu_util import assert_parity, check_output, ref_of, run_gpu

pytestmark = pytest.mark.gpu

OPS = ["softmax", "rmsnorm", "layernorm", "cross_entropy"]
EPS = {"softmax": None, "rmsnorm": 1e-6, "layernorm": 1e-5, "cross_entropy": None}
GEN = {"softmax": dict(std=4.0), "rmsnorm": {}, "layernorm": dict(mean=3.0, std=2.0),
       "cross_entropy": {}}

WORKLOAD_CASES = [(name, pol) for name, w in synth.WORKLOADS.items() for pol in w["policies"]]


@pytest.mark.parametrize("name,policy", WORKLOAD_CASES, ids=[f"{n}-{p}" for n, p in WORKLOAD_CASES])
def test_workload_parity(name, policy):
    w = synth.WORKLOADS[name]
    print(f"\n[gpu] workload {name} policy={policy}", flush=True)
    inp = synth.workload_inputs(name)
    got, st, _ = run_gpu(w["op"], inp, w["eps"], policy)
    assert st == lr.LR_OK, lr.lr_status_string(st)
    ref = ref_of(w["op"], inp, w["eps"])
    worst = assert_parity(got, ref, name)
    if policy == "ordered_fold":
        check_output(w["op"], inp, w["eps"], policy, got, name)
    print(f"[gpu] {name} {policy}: worst err/bound = {worst:.3g}", flush=True)


RAGGED_COLS = [1, 2, 3, 4, 5, 7, 8, 31, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1023, 1024, 1025, 1537,
               4096, 12289]
RAGGED_ROWS = [1, 2, 7, 17, 37]


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("policy", ["unordered_tree", "ordered_fold"])
def test_ragged_sweep(op, policy):
    print(f"\n[gpu] ragged sweep {op} {policy}", flush=True)
    for cols in RAGGED_COLS:
        for rows in RAGGED_ROWS:
            inp = synth.make_inputs(op, rows, cols, seed=cols * 131 + rows, **GEN[op])
            got, st, _ = run_gpu(op, inp, EPS[op], policy)
            assert st == lr.LR_OK
            check_output(op, inp, EPS[op], policy, got, f"{op} {rows}x{cols}")


FORCED_SHAPES = [(17, 257), (37, 1537), (7, 4096), (3, 12289), (5, 64), (2, 6144)]


@pytest.mark.parametrize("op", OPS)
def test_every_legal_plan_forced(op):
    facts = lr.lr_device_facts_query()
    n = 0
    for rows, cols in FORCED_SHAPES:
        inp = synth.make_inputs(op, rows, cols, seed=rows + cols, **GEN[op])
        for policy in ("unordered_tree", "ordered_fold"):
            plans = lr.lr_plan_enumerate(facts, op, rows, cols, policy, 1 if cols % 4 == 0 else 0)
            assert plans
            print(f"\n[gpu] forced plans {op} {rows}x{cols} {policy}: {len(plans)}", flush=True)
            for p in plans:
                got, st, _ = run_gpu(op, inp, EPS[op], policy, plan=p)
                assert st == lr.LR_OK, (p, lr.lr_status_string(st))
                check_output(op, inp, EPS[op], policy, got, f"{op} {rows}x{cols} {p}")
                n += 1
    assert n > 50


@pytest.mark.parametrize("op", ["softmax", "rmsnorm", "layernorm"])
def test_canary_padding_untouched_every_plan(op):
    facts = lr.lr_device_facts_query()
    rows, cols, pad = 9, 1030, 37
    inp = synth.make_inputs(op, rows, cols, seed=11, **GEN[op])
    canary = -12345.5
    for policy in ("unordered_tree", "ordered_fold"):
        for p in lr.lr_plan_enumerate(facts, op, rows, cols, policy, 0):
            got, st, ex = run_gpu(op, inp, EPS[op], policy, plan=p, x_pad=3, y_pad=pad, canary=canary)
            assert st == lr.LR_OK
            check_output(op, inp, EPS[op], policy, got, f"{op} canary {p}")
            full = ex["yfull"]
            assert (full[:pad] == canary).all() and (full[pad + rows * cols:] == canary).all(), p


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("x_pad,y_pad", [(1, 0), (2, 2), (3, 1), (0, 3)])
def test_misaligned_bases(op, x_pad, y_pad):
    for rows, cols in [(6, 4096), (5, 1537), (3, 63)]:
        inp = synth.make_inputs(op, rows, cols, seed=x_pad * 7 + y_pad, **GEN[op])
        for policy in ("unordered_tree", "ordered_fold"):
            got, st, _ = run_gpu(op, inp, EPS[op], policy, x_pad=x_pad, y_pad=y_pad)
            assert st == lr.LR_OK
            check_output(op, inp, EPS[op], policy, got, f"{op} {rows}x{cols} pads {x_pad},{y_pad}")


@pytest.mark.parametrize("op", ["softmax", "rmsnorm", "layernorm"])
def test_in_place(op):
    for rows, cols in [(37, 1537), (64, 6144)]:
        inp = synth.make_inputs(op, rows, cols, seed=3, **GEN[op])
        for policy in ("unordered_tree", "ordered_fold"):
            got, st, _ = run_gpu(op, inp, EPS[op], policy, in_place=True)
            assert st == lr.LR_OK
            check_output(op, inp, EPS[op], policy, got, f"{op} in place")


def test_parameters_omitted():
    rows, cols = 33, 2050
    x = synth.normal_f32(1, 0, rows * cols, 3.0, 2.0).reshape(rows, cols)
    for policy in ("unordered_tree", "ordered_fold"):
        got, st, _ = run_gpu("rmsnorm", {"x": x}, 1e-6, policy)
        assert st == lr.LR_OK
        check_output("rmsnorm", {"x": x}, 1e-6, policy, got, "rmsnorm no gamma")
        got, st, _ = run_gpu("layernorm", {"x": x}, 1e-5, policy)
        assert st == lr.LR_OK
        check_output("layernorm", {"x": x}, 1e-5, policy, got, "layernorm no affine")


def test_softmax_dyadic_shift_bit_identical():
    # x = k/64 and an integer shift: x + c and x - max are exact in FP32, so the
    # GPU output must not change by a single bit
    rng = np.random.default_rng(9)
    x = (rng.integers(-1024, 1025, size=(37, 1537)) / 64.0).astype(np.float32)
    base, _, _ = run_gpu("softmax", {"x": x})
    for c in (1.0, 64.0, -1000.0):
        got, _, _ = run_gpu("softmax", {"x": x + np.float32(c)})
        assert np.array_equal(got.view(np.uint32), base.view(np.uint32))
    np.testing.assert_allclose(base.astype(np.float64).sum(axis=1), 1.0, atol=1e-5)


def test_norm_closed_forms_on_gpu():
    g = synth.uniform_f32(0, 1, 4096, 0.5, 1.5)
    x = np.full((4, 4096), -2.0, dtype=np.float32)
    got, _, _ = run_gpu("rmsnorm", {"x": x, "gamma": g}, 0.0)
    np.testing.assert_allclose(got, np.tile(-g, (4, 1)), rtol=1e-6)
    x = synth.normal_f32(2, 0, 8 * 6144, 3.0, 2.0).reshape(8, 6144)
    got, _, _ = run_gpu("layernorm", {"x": x}, 0.0)
    y = got.astype(np.float64)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-6)
    np.testing.assert_allclose(y.var(axis=1), 1.0, rtol=1e-5)


def test_cross_entropy_matches_minus_log_softmax_on_gpu():
    inp = synth.cross_entropy_inputs(64, 4099, seed=5)
    loss, _, _ = run_gpu("cross_entropy", inp)
    p, _, _ = run_gpu("softmax", {"x": inp["logits"]})
    sel = p[np.arange(64), inp["labels"]].astype(np.float64)
    np.testing.assert_allclose(loss, -np.log(sel), rtol=1e-4, atol=1e-5)
