"""The ordered policies on the GPU against the hand-worked FP32 results of
tests/golden/ordered_post_fold.json (the steps after the fold: the mean as
acc / cols, IEEE division and square root, (x * r) * gamma and
((x - mu) * r) * gamma + beta, each rounded on its own; "TIRx Metal reduction
lowering", section 1: ordered reductions keep the serial path and need
precise math).  Every legal plan of each ordered policy must give the
golden bits; the rows are repeated so that several rows share a launch."""
import json
import os

import numpy as np
import pytest
import torch

import row_reductions_amd as lr
from gpu_util import DEV

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ordered_post_fold.json")
POLICIES = ["ordered_fold", "ordered_tree", "fold_right"]


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _vec(v):
    return None if v is None else torch.tensor(v, dtype=torch.float32, device=DEV)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_ordered_policies_give_the_hand_worked_bits(case):
    rows = 5
    x = np.tile(np.array(case["x"], dtype=np.float32), (rows, 1))
    cols = x.shape[1]
    want = np.tile(np.array(case["expected"], dtype=np.float32), (rows, 1)).view(np.uint32)
    xd = torch.from_numpy(x).to(DEV)
    g = _vec(case.get("gamma"))
    b = _vec(case.get("beta"))
    facts = lr.lr_device_facts_query()
    n = 0
    for pol in POLICIES:
        plans = [None] + list(lr.lr_plan_enumerate(facts, case["op"], rows, cols, pol, 1 if cols % 4 == 0 else 0))
        for p in plans:
            y = torch.full_like(xd, float("nan"))
            if case["op"] == "rmsnorm":
                st = lr.lr_rmsnorm_f32(xd, g, y, rows, cols, case["eps"], pol, plan=p)
            else:
                st = lr.lr_layernorm_f32(xd, g, b, y, rows, cols, case["eps"], pol, plan=p)
            assert st == lr.LR_OK, (pol, p, lr.lr_status_string(st))
            torch.cuda.synchronize()
            got = y.cpu().numpy().view(np.uint32)
            bad = np.argwhere(got != want)
            assert bad.size == 0, (case["name"], pol, p, tuple(bad[0]),
                                   y.cpu().numpy()[tuple(bad[0])], np.float32(case["expected"][bad[0][1]]))
            n += 1
    assert n >= len(POLICIES) * 2
