"""Property tests of the planner on the CPU (hypothesis): any plan that
lr_plan_validate accepts -- enumerated, automatic or arbitrary field values
-- covers each (row, element) of the problem exactly once in the host replay
of the kernels' index functions ("TIRx Metal reduction lowering", section
4.4), whatever the row phase; and validation accepts or rejects, it never
repairs a plan."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import row_reductions_amd as lr

F = lr.lr_device_facts_mi355x()
OPS = ["softmax", "rmsnorm", "layernorm", "cross_entropy", "add_layernorm", "row_sum", "row_minmax"]
POLICIES = ["unordered_tree", "ordered_fold", "ordered_tree", "fold_right"]
FAMILIES = [lr.LR_FAMILY_CACHE, lr.LR_FAMILY_STREAM, lr.LR_FAMILY_ORDERED, lr.LR_FAMILY_TREE, lr.LR_FAMILY_SPLIT]

SETTINGS = settings(max_examples=600, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def covered_once(plan, rows, cols, aligned):
    for phase in ((0,) if aligned else (0, 1, 2, 3)):
        counts = np.zeros(rows * cols, dtype=np.uint32)
        assert lr.lr_coverage_check(plan, rows, cols, phase, counts.ctypes.data) == lr.LR_OK
        if not (counts == 1).all():
            return False
    return True


def make_plan(family, S, Q, vec, nch, blocks, splits, lanes=0):
    """lanes: 4 .. 32 for a sub-wave team (lanes * Q threads), else whole waves"""
    p = lr.LrPlan()
    p.family, p.waves_per_row, p.rows_per_block, p.vec = family, S, Q, vec
    p.chunks_per_lane, p.blocks, p.splits = nch, blocks, splits
    p.threads_per_block = lanes * Q if lanes else 64 * S * Q
    p.lanes_per_row = lanes if lanes else 64 * S
    return p


problems = st.tuples(st.sampled_from(OPS), st.integers(1, 5), st.integers(1, 4096), st.sampled_from(POLICIES),
                     st.booleans())


ALLOWED = {  # families each policy may run on
    "unordered_tree": [lr.LR_FAMILY_CACHE, lr.LR_FAMILY_STREAM, lr.LR_FAMILY_SPLIT],
    "ordered_fold": [lr.LR_FAMILY_ORDERED],
    "fold_right": [lr.LR_FAMILY_ORDERED],
    "ordered_tree": [lr.LR_FAMILY_TREE, lr.LR_FAMILY_ORDERED],
}
CACHE_CHUNKS = [1, 2, 3, 4, 6, 8, 12, 16, 24, 32]
CHUNKS = {lr.LR_FAMILY_CACHE: CACHE_CHUNKS, lr.LR_FAMILY_TREE: CACHE_CHUNKS, lr.LR_FAMILY_SPLIT: [1, 2, 3, 4, 6, 8],
          lr.LR_FAMILY_STREAM: [4], lr.LR_FAMILY_ORDERED: [0]}


@SETTINGS
@given(problems, st.data())
def test_any_accepted_plan_covers_each_element_once(problem, data):
    """plans drawn near the legal set (each field off its family's values now
    and then), so that many are accepted and every accepted one is checked"""
    op, rows, cols, policy, want_aligned = problem
    aligned = 1 if want_aligned and cols % 4 == 0 else 0
    off = lambda: data.draw(st.integers(0, 9)) == 0  # noqa: E731
    family = data.draw(st.sampled_from(FAMILIES if off() else ALLOWED[policy]))
    # few waves per row make stripes of several chunks, where the boundary is
    S = 1 if family == lr.LR_FAMILY_ORDERED and not off() else data.draw(st.one_of(st.integers(1, 3),
                                                                                     st.integers(1, 16)))
    Q = 1 if family == lr.LR_FAMILY_SPLIT and not off() else data.draw(st.integers(1, 16 // S))
    vec = (1 if family == lr.LR_FAMILY_ORDERED else 4) if not off() else data.draw(st.sampled_from([1, 2, 4]))
    splits = 0
    if family == lr.LR_FAMILY_SPLIT or off():
        splits = data.draw(st.sampled_from([1, 2, 3, 4, 8, 16, 32, 64, 65]))
    # chunks per lane mostly at the legality boundary: the compiled instance
    # just below the stripe the row needs, the one that covers it, the next
    inst = CHUNKS[family]
    nv = cols // 4 if aligned else (cols + 6) // 4
    if family == lr.LR_FAMILY_SPLIT and splits >= 1:
        nv = -(-nv // splits)
    need = -(-nv // (64 * S))
    near = [c for c in inst if c < need][-1:] + [c for c in inst if c >= need][:2]
    if off():
        nch = data.draw(st.sampled_from([0, 1, 5, 7, 9, 64]))
    else:
        nch = data.draw(st.sampled_from(near or inst))
    blocks = rows * splits if family == lr.LR_FAMILY_SPLIT else -(-rows // Q)
    if off():
        blocks += data.draw(st.sampled_from([1, -1]))
    p = make_plan(family, S, Q, vec, nch, blocks, splits)
    before = bytes(p)
    st_ = lr.lr_plan_validate(F, op, rows, cols, policy, aligned, p)
    assert bytes(p) == before  # validation never edits the plan
    assert st_ in (lr.LR_OK, lr.LR_ERR_UNREALIZABLE_PLAN)
    if st_ == lr.LR_OK:
        assert p.threads_per_block <= 1024 and p.blocks >= 1
        assert covered_once(p, rows, cols, aligned), (op, rows, cols, policy, aligned, p)


@SETTINGS
@given(problems)
def test_every_enumerated_and_automatic_plan_is_accepted_and_covers(problem):
    op, rows, cols, policy, want_aligned = problem
    aligned = 1 if want_aligned and cols % 4 == 0 else 0
    plans = lr.lr_plan_enumerate(F, op, rows, cols, policy, aligned)
    assert plans
    plans.append(lr.lr_plan_for_device(F, op, rows, cols, policy, aligned))
    plans.append(lr.lr_plan_for_device_ws(F, op, rows, cols, policy, aligned))
    # a sample of the enumerated plans keeps the example fast
    for p in plans[:: max(1, len(plans) // 12)] + plans[-2:]:
        assert lr.lr_plan_validate(F, op, rows, cols, policy, aligned, p) == lr.LR_OK
        assert covered_once(p, rows, cols, aligned), (op, rows, cols, policy, aligned, p)


@SETTINGS
@given(st.sampled_from(OPS), st.integers(1, 300), st.integers(1, 300), st.booleans(), st.data())
def test_accepted_sub_wave_plans_cover_each_element_once(op, rows, cols, want_aligned, data):
    """sub-wave CACHE plans near the boundary of legality: team width, waves
    per workgroup (whole or not), stripe; part-empty waves and workgroups"""
    aligned = 1 if want_aligned and cols % 4 == 0 else 0
    tree = data.draw(st.booleans())  # TREE plans (ordered_tree) or CACHE (unordered)
    family, policy = (lr.LR_FAMILY_TREE, "ordered_tree") if tree else (lr.LR_FAMILY_CACHE, "unordered_tree")
    L = data.draw(st.sampled_from([4, 8, 16, 32]))
    per_wave = 64 // L
    Q = data.draw(st.one_of(st.integers(1, 16).map(lambda w: w * per_wave), st.integers(1, 1024 // L + 1)))
    nv = cols // 4 if aligned else (cols + 6) // 4
    need = -(-nv // L)
    nch = data.draw(st.sampled_from([c for c in (1, 2, 3) if c >= need - 1] or [1]))
    p = make_plan(family, 1, Q, 4, nch, -(-rows // Q), 0, L)
    if lr.lr_plan_validate(F, op, rows, cols, policy, aligned, p) == lr.LR_OK:
        assert Q % per_wave == 0 and L * Q <= 1024 and nch in (1, 2) and nch >= need
        assert not tree or (aligned and nch == 1)
        assert covered_once(p, rows, cols, aligned), (op, rows, cols, aligned, p)


@SETTINGS
@given(st.sampled_from(OPS), st.integers(1, 4), st.integers(8, 8192), st.booleans(), st.data())
def test_accepted_split_plans_cover_each_element_once(op, rows, cols, want_aligned, data):
    """split-row plans near the boundary of legality: segments and stripes"""
    aligned = 1 if want_aligned and cols % 4 == 0 else 0
    G = data.draw(st.sampled_from([2, 3, 4, 8, 16, 64]))
    S = data.draw(st.one_of(st.integers(1, 2), st.integers(1, 16)))
    nv = -(-(cols // 4 if aligned else (cols + 6) // 4) // G)
    need = -(-nv // (64 * S))
    inst = CHUNKS[lr.LR_FAMILY_SPLIT]
    nch = data.draw(st.sampled_from(([c for c in inst if c < need][-1:] + [c for c in inst if c >= need][:2]) or inst))
    p = make_plan(lr.LR_FAMILY_SPLIT, S, 1, 4, nch, rows * G, G)
    if lr.lr_plan_validate(F, op, rows, cols, "unordered_tree", aligned, p) == lr.LR_OK:
        assert nch >= need and G <= -(-cols // 4)
        assert covered_once(p, rows, cols, aligned), (op, rows, cols, aligned, p)


@SETTINGS
@given(st.sampled_from(OPS), st.integers(1, 400), st.integers(1, 80), st.booleans(), st.data())
def test_accepted_lane_plans_cover_each_element_once(op, rows, cols, want_aligned, data):
    """one-lane-per-row plans (ORDERED, lanes_per_row 1) near the boundary of
    legality: lanes per workgroup (one wavefront is legal), compiled and
    uncompiled stripes, aligned and misaligned rows"""
    aligned = 1 if want_aligned and cols % 4 == 0 else 0
    policy = data.draw(st.sampled_from(["ordered_fold", "fold_right", "ordered_tree"]))
    Q = data.draw(st.one_of(st.sampled_from([64, 128, 192, 256, 320]), st.integers(1, 300)))
    nch = data.draw(st.sampled_from([0, 1, 2, 3, 4, 8, 16, 32]))
    p = make_plan(lr.LR_FAMILY_ORDERED, 1, Q, 1, nch, -(-rows // Q), 0, 1)
    if lr.lr_plan_validate(F, op, rows, cols, policy, aligned, p) == lr.LR_OK:
        assert Q == 64 and nch in (1, 2, 4, 8, 16) and 4 * nch >= cols
        assert covered_once(p, rows, cols, aligned), (op, rows, cols, p)
