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
from gpu_util import ATOL, DEV, RTOL, assert_parity, guards_intact, placed

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
