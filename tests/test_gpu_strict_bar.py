"""GPU parity of the deterministic policies on the five workloads at full size,
at the strict bar |gpu - ref| <= 1e-6 + 1e-5 |ref| against the double
oracle, with every launch giving the same bits.

The policy tests elsewhere check the ordered policies against their FP32
replays (RMSNorm, LayerNorm: bit for bit) or, for softmax and cross-entropy
on arbitrary shapes, against the bar widened by the serial-sum bound.  Here
the workloads themselves are held to the unwidened bar under ordered_fold,
ordered_tree and fold_right.  Every pair meets it but one: LayerNorm
64x12289 (x ~ N(3, 2^2)) under the two serial folds, where the FP32 left or
right fold of 12289 values near 3 rounds the row's mean by about 1e-5 and
outputs near zero miss the bar by up to about 10x.  That error belongs to
the fold order itself, not to the kernels: for those two pairs the test
requires the GPU result to equal the oracle's FP32 replay of the same fold
bit for bit, and checks that the replay misses the bar just as much."""
import numpy as np
import pytest

import oracle
import row_reductions_amd as lr
import synth
from gpu_util import assert_parity, ref_of, run_gpu, within_bar

pytestmark = pytest.mark.gpu

POLICIES = ("ordered_fold", "ordered_tree", "fold_right")
# (workload, policy) pairs whose FP32 serial fold is itself outside the bar
SERIAL_FOLD_OUTSIDE_BAR = {("layernorm_64x12289", "ordered_fold"), ("layernorm_64x12289", "fold_right")}


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_strict_bar_deterministic_policies(name):
    w = synth.WORKLOADS[name]
    inp = synth.workload_inputs(name)
    ref = ref_of(w["op"], inp, w["eps"])
    for policy in POLICIES:
        print(f"\n[gpu] strict bar {name} {policy}", flush=True)
        got, st, _ = run_gpu(w["op"], inp, w["eps"], policy)
        assert st == lr.LR_OK, lr.lr_status_string(st)
        again, st, _ = run_gpu(w["op"], inp, w["eps"], policy)
        assert st == lr.LR_OK
        assert np.array_equal(got.view(np.uint32), again.view(np.uint32)), f"{name} [{policy}]: launches differ"
        if (name, policy) in SERIAL_FOLD_OUTSIDE_BAR:
            rep = oracle.layernorm_ordered_f32(inp["x"], inp["gamma"], inp["beta"], w["eps"], policy=policy)
            assert np.array_equal(got.view(np.uint32), rep.view(np.uint32)), \
                f"{name} [{policy}]: differs from the FP32 replay of the fold"
            ok, worst = within_bar(rep, ref)
            assert not ok, f"{name} [{policy}]: the replay now meets the bar; drop the exemption"
            print(f"[gpu] {name} {policy}: equal to the FP32 replay, whose worst err/bound is {worst:.3g}",
                  flush=True)
            continue
        worst = assert_parity(got, ref, f"{name} [{policy}]")
        print(f"[gpu] {name} {policy}: worst err/bound = {worst:.3g}", flush=True)
