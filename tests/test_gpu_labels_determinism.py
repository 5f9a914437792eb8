"""GPU: exact label indexing of the guarded cross-entropy gather, and
determinism (ordered_fold bit-identical across launches and, for RMSNorm and
LayerNorm, bit-equal to the CPU FP32 replay; unordered_tree bit-identical
across launches of one plan)."""
import numpy as np
import pytest
import torch

import oracle
import row_reductions_amd as lr
import synth
from gpu_util import DEV, assert_parity, check_output, ref_of, run_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("policy", ["unordered_tree", "ordered_fold"])
def test_ramp_logits_make_index_errors_exact(policy):
    # x[r, j] = j * 2^-8: a label off by k changes the loss by exactly k * 2^-8
    cols = 4096
    rows = 64
    x = np.tile((np.arange(cols) * 2.0 ** -8).astype(np.float32), (rows, 1))
    lab = synth.labels_i64(7, 3, rows, 0, cols)
    lab[:4] = [0, 1, cols - 2, cols - 1]
    got, st, _ = run_gpu("cross_entropy", {"logits": x, "labels": lab}, policy=policy)
    assert st == lr.LR_OK
    check_output("cross_entropy", {"logits": x, "labels": lab}, None, policy, got, "ramp")
    # the loss differences between rows pin the selected index exactly
    d = (got.astype(np.float64) - got[0]) / 2.0 ** -8
    np.testing.assert_allclose(d, -(lab - lab[0]).astype(np.float64), atol=0.02)


@pytest.mark.parametrize("policy", ["unordered_tree", "ordered_fold"])
def test_out_of_range_labels_select_zero(policy):
    cols = 4096
    bad = [-1, cols, 2 ** 31, 2 ** 32 + 3, -(2 ** 63), 2 ** 63 - 1, 2 ** 32 + 5, -(2 ** 32) + 7]
    rows = len(bad)
    inp = synth.cross_entropy_inputs(rows, cols, seed=2)
    inp["labels"] = np.array(bad, dtype=np.int64)
    got, st, _ = run_gpu("cross_entropy", inp, policy=policy)
    assert st == lr.LR_OK
    check_output("cross_entropy", inp, None, policy, got, "guard")
    # = logsumexp of the row (the fill value 0 is selected)
    x = inp["logits"].astype(np.float64)
    m = x.max(axis=1)
    lse = m + np.log(np.exp(x - m[:, None]).sum(axis=1))
    np.testing.assert_allclose(got, lse, rtol=1e-5)


def test_cross_entropy_7x4096_every_row():
    # the pages' cross-entropy test shape: every loss checked
    inp = synth.cross_entropy_inputs(7, 4096, seed=0)
    for policy in ("unordered_tree", "ordered_fold"):
        got, st, _ = run_gpu("cross_entropy", inp, policy=policy)
        assert st == lr.LR_OK
        check_output("cross_entropy", inp, None, policy, got, "7x4096")


def _launch_many(op, inp, eps, policy, n, plan=None):
    x = inp["logits"] if op == "cross_entropy" else inp["x"]
    rows, cols = x.shape
    xd = torch.from_numpy(x).to(DEV)
    g = torch.from_numpy(inp["gamma"]).to(DEV) if "gamma" in inp else None
    b = torch.from_numpy(inp["beta"]).to(DEV) if "beta" in inp else None
    outs = []
    for _ in range(n):
        if op == "cross_entropy":
            y = torch.empty(rows, device=DEV)
            st = lr.lr_cross_entropy_f32(xd, torch.from_numpy(inp["labels"]).to(DEV), y, rows, cols, policy,
                                         plan=plan)
        else:
            y = torch.empty(rows, cols, device=DEV)
            if op == "softmax":
                st = lr.lr_softmax_f32(xd, y, rows, cols, policy, plan=plan)
            elif op == "rmsnorm":
                st = lr.lr_rmsnorm_f32(xd, g, y, rows, cols, eps, policy, plan=plan)
            else:
                st = lr.lr_layernorm_f32(xd, g, b, y, rows, cols, eps, policy, plan=plan)
        assert st == lr.LR_OK
        outs.append(y)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


@pytest.mark.parametrize("op,eps", [("softmax", None), ("rmsnorm", 1e-6), ("layernorm", 1e-5),
                                    ("cross_entropy", None)])
def test_ordered_fold_bit_identical_across_launches(op, eps):
    inp = synth.make_inputs(op, 256, 3072, seed=0)
    outs = _launch_many(op, inp, eps, "ordered_fold", 20)
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    check_output(op, inp, eps, "ordered_fold", outs[0], f"{op} ordered")


@pytest.mark.parametrize("rows,cols", [(256, 3072), (37, 1537), (5, 12289), (3, 1)])
def test_ordered_fold_equals_cpu_fp32_replay(rows, cols):
    inp = synth.rmsnorm_inputs(rows, cols, seed=1)
    got = _launch_many("rmsnorm", inp, 1e-6, "ordered_fold", 1)[0]
    rep = oracle.rmsnorm_fold_f32(inp["x"], inp["gamma"], 1e-6)
    assert np.array_equal(got.view(np.uint32), rep.view(np.uint32)), "rmsnorm ordered != FP32 replay"
    inp = synth.layernorm_inputs(rows, cols, seed=1, mean=3.0, std=2.0)
    got = _launch_many("layernorm", inp, 1e-5, "ordered_fold", 1)[0]
    rep = oracle.layernorm_fold_f32(inp["x"], inp["gamma"], inp["beta"], 1e-5)
    assert np.array_equal(got.view(np.uint32), rep.view(np.uint32)), "layernorm ordered != FP32 replay"


def test_ordered_fold_is_plan_independent():
    facts = lr.lr_device_facts_query()
    inp = synth.layernorm_inputs(40, 1000, seed=3)
    outs = []
    for p in lr.lr_plan_enumerate(facts, "layernorm", 40, 1000, "ordered_fold", 1):
        outs.append(_launch_many("layernorm", inp, 1e-5, "ordered_fold", 1, plan=p)[0])
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))


@pytest.mark.parametrize("op,eps", [("softmax", None), ("rmsnorm", 1e-6), ("layernorm", 1e-5),
                                    ("cross_entropy", None)])
def test_unordered_same_plan_bit_identical(op, eps):
    inp = synth.make_inputs(op, 768, 6144 if op != "cross_entropy" else 8000, seed=0)
    outs = _launch_many(op, inp, eps, "unordered_tree", 20)
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
