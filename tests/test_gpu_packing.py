"""Packing of cooperating rows on the GPU ("TIRx Metal reduction lowering",
section 4.3: Q rows of S > 1 waves share one workgroup).  Thirty-six
configurations, as in the pages' packing tests: row sum, softmax, LayerNorm
without affine, and row minimum with maximum, each under nine packed plans.
The plans cover non-power-of-two S and widths, the register (CACHE) and
reload (STREAM) families, ragged row counts that leave inactive teams in the
last workgroup, 1024-thread workgroups and the planner's own width for a
fixed Q.  Every tensor sits between guard rows: input guards hold values
that would change any result they leaked into, output guards hold a
sentinel that must survive."""
import numpy as np
import pytest
import torch

import oracle
import row_reductions_amd as lr
import synth
from gpu_util import DEV, assert_parity

pytestmark = pytest.mark.gpu

GUARD = 3          # guard rows on each side of every tensor
SENTINEL = -7.25   # output guard value
POISON = 1.0e30    # input guard value

# (family, S, Q, rows, cols); S = None: the first legal width S > 1 for that
# Q.  Every row count leaves a ragged last workgroup (rows % Q != 0).
CONFIGS = [
    ("cache", 2, 2, 5, 1000),
    ("cache", 3, 2, 7, 1537),
    ("cache", 2, 3, 8, 3000),
    ("cache", 5, 3, 10, 4097),
    ("cache", 4, 4, 9, 2049),     # 1024 threads
    ("stream", 3, 5, 11, 1537),   # 960 threads
    ("stream", 2, 4, 6, 12289),
    ("cache", 8, 2, 3, 6000),     # 1024 threads, one inactive team
    ("cache", None, 4, 13, 700),
]
OPS = ["row_sum", "softmax", "layernorm", "row_minmax"]


def packed_plan(op, family, S, Q, rows, cols):
    facts = lr.lr_device_facts_query()
    fam = {"cache": lr.LR_FAMILY_CACHE, "stream": lr.LR_FAMILY_STREAM}[family]
    for p in lr.lr_plan_enumerate(facts, op, rows, cols, "unordered_tree", 1 if cols % 4 == 0 else 0):
        if p.family == fam and p.rows_per_block == Q and p.waves_per_row > 1 and (S is None or p.waves_per_row == S):
            return p
    raise AssertionError(f"no legal {family} plan S={S} Q={Q} for {rows}x{cols}")


def guarded(a, fill):
    """`a` (rows x cols) between GUARD rows of `fill` on each side; returns
    (view of the rows, whole buffer)."""
    rows, cols = a.shape
    full = torch.full((rows + 2 * GUARD, cols), fill, dtype=torch.float32, device=DEV)
    full[GUARD:GUARD + rows].copy_(torch.from_numpy(np.ascontiguousarray(a)))
    return full[GUARD:GUARD + rows], full


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("cfg", CONFIGS, ids=[f"{c[0]}-S{c[1]}-Q{c[2]}-{c[3]}x{c[4]}" for c in CONFIGS])
def test_packed_cooperating_rows(op, cfg):
    family, S, Q, rows, cols = cfg
    plan = packed_plan(op, family, S, Q, rows, cols)
    assert Q > 1 and plan.waves_per_row > 1 and rows % Q != 0
    print(f"\n[gpu] packing {op} {rows}x{cols} {plan}", flush=True)
    x = synth.normal_f32(rows * 31 + cols, 0, rows * cols, 0.5, 2.0).reshape(rows, cols)
    xv, _ = guarded(x, POISON)
    if op in ("softmax", "layernorm"):
        yv, yfull = guarded(np.full_like(x, SENTINEL), SENTINEL)
        if op == "softmax":
            st = lr.lr_softmax_f32(xv, yv, rows, cols, plan=plan)
            ref = oracle.softmax(x)
        else:
            st = lr.lr_layernorm_f32(xv, None, None, yv, rows, cols, 1e-5, plan=plan)
            ref = oracle.layernorm(x, None, None, 1e-5)
        torch.cuda.synchronize()
        assert st == lr.LR_OK, lr.lr_status_string(st)
        full = yfull.cpu().numpy()
        assert (full[:GUARD] == SENTINEL).all() and (full[GUARD + rows:] == SENTINEL).all(), "guard rows written"
        assert_parity(full[GUARD:GUARD + rows], ref, f"{op} {cfg}")
        return
    outs = [torch.full((rows + 2 * GUARD,), SENTINEL, device=DEV) for _ in range(2)]
    views = [o[GUARD:GUARD + rows] for o in outs]
    if op == "row_sum":
        st = lr.lr_row_sum_f32(xv, views[0], rows, cols, plan=plan)
    else:
        st = lr.lr_row_minmax_f32(xv, views[0], views[1], rows, cols, plan=plan)
    torch.cuda.synchronize()
    assert st == lr.LR_OK, lr.lr_status_string(st)
    got = [o.cpu().numpy() for o in outs]
    for g in got[: 1 if op == "row_sum" else 2]:
        assert (g[:GUARD] == SENTINEL).all() and (g[GUARD + rows:] == SENTINEL).all(), "guard entries written"
    if op == "row_sum":
        ref = oracle.row_sum(x)
        bound = 1e-6 + 1e-5 * np.abs(x.astype(np.float64)).sum(axis=1)
        assert (np.abs(got[0][GUARD:GUARD + rows] - ref) <= bound).all(), cfg
    else:
        lo, hi = oracle.row_minmax(x)
        assert np.array_equal(got[0][GUARD:GUARD + rows], lo) and np.array_equal(got[1][GUARD:GUARD + rows], hi)


def test_configs_include_full_workgroups():
    """1024-thread workgroups (S * Q = 16 waves) are among the configurations"""
    assert any(S is not None and 64 * S * Q == 1024 for _, S, Q, _, _ in CONFIGS)
