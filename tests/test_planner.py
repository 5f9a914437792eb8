"""Planner on the CPU: every legal plan covers each (row, element) exactly
once (the coverage requirement of "TIRx Metal reduction lowering", section
4.4, checked by replaying the kernels' own index functions), plans respect
the device limits, explicit plans are honoured or rejected but never
clamped, and the automatic choice is deterministic."""
import ctypes

import numpy as np
import pytest

import row_reductions_amd as lr

F = lr.lr_device_facts_mi355x()
OPS = ["softmax", "rmsnorm", "layernorm", "cross_entropy", "add_layernorm", "row_sum", "row_minmax"]

WIDTHS = list(range(1, 131)) + [255, 256, 257, 511, 513, 1023, 1024, 1025, 1537, 3072, 6144, 12289]


def coverage(plan, rows, cols, phase):
    counts = np.zeros(rows * cols, dtype=np.uint32)
    st = lr.lr_coverage_check(plan, rows, cols, phase, counts.ctypes.data)
    assert st == lr.LR_OK
    return counts


POLICIES = ["unordered_tree", "ordered_fold", "ordered_tree", "fold_right"]


@pytest.mark.parametrize("policy", POLICIES)
def test_every_plan_covers_each_element_once(policy):
    checked = 0
    for cols in WIDTHS:
        rows = 5 if cols < 2000 else 2
        aligned_opts = (1, 0) if cols % 4 == 0 else (0,)
        for aligned in aligned_opts:
            plans = lr.lr_plan_enumerate(F, "softmax", rows, cols, policy, aligned)
            assert plans, (cols, aligned)
            phases = (0,) if aligned else (0, 1, 2, 3)
            for p in plans:
                for ph in phases:
                    c = coverage(p, rows, cols, ph)
                    assert (c == 1).all(), (cols, aligned, ph, p)
                    checked += 1
    assert checked > 1000


def test_config_shapes_every_plan_covers_once():
    for rows, cols in [(37, 1537), (256, 3072), (64, 12289), (3, 6144), (2, 32000)]:
        aligned = 1 if cols % 4 == 0 else 0
        for p in lr.lr_plan_enumerate(F, "cross_entropy", rows, cols, "unordered_tree", aligned):
            for ph in ((0,) if aligned else (0, 3)):
                assert (coverage(p, rows, cols, ph) == 1).all(), (rows, cols, p)


def test_plans_respect_device_limits():
    for op in OPS:
        for rows, cols in [(1, 1), (37, 1537), (768, 6144), (4096, 32000), (5, 100000)]:
            for policy in POLICIES:
                for p in lr.lr_plan_enumerate(F, op, rows, cols, policy, 1 if cols % 4 == 0 else 0):
                    if p.lanes_per_row == 1:  # one lane per row: ORDERED, one wavefront of 64 rows
                        assert p.family == lr.LR_FAMILY_ORDERED and p.waves_per_row == 1
                        assert p.rows_per_block == p.threads_per_block == 64 and p.chunks_per_lane in (1, 2, 4, 8, 16)
                        assert 4 * p.chunks_per_lane >= cols and p.lds_bytes == 64 * (4 * p.chunks_per_lane + 2) * 4
                    elif p.lanes_per_row < 64:  # sub-wave teams: CACHE or TREE, one wave's lanes shared by rows
                        assert p.family in (lr.LR_FAMILY_CACHE, lr.LR_FAMILY_TREE) and p.waves_per_row == 1
                        assert p.lanes_per_row in (4, 8, 16, 32) and p.rows_per_block % (64 // p.lanes_per_row) == 0
                        assert p.threads_per_block == p.lanes_per_row * p.rows_per_block <= 1024
                        assert p.chunks_per_lane in (1, 2)
                    else:
                        assert p.lanes_per_row == 64 * p.waves_per_row
                        assert p.threads_per_block == 64 * p.waves_per_row * p.rows_per_block <= 1024
                    if p.family == lr.LR_FAMILY_SPLIT:
                        assert p.rows_per_block == 1 and 2 <= p.splits <= 64
                        assert p.blocks == rows * p.splits
                        seg = -(-((cols + 6) // 4 if cols % 4 else cols // 4) // p.splits)
                        assert p.chunks_per_lane in (1, 2, 3, 4, 6, 8)
                        assert p.chunks_per_lane * 64 * p.waves_per_row >= seg
                        assert lr.lr_plan_workspace_bytes(p, rows) == rows * p.splits * 8
                    else:
                        assert p.splits == 0 and lr.lr_plan_workspace_bytes(p, rows) == 0
                        assert p.blocks == -(-rows // p.rows_per_block)
                    assert p.lds_bytes <= 64 * 1024
                    if p.family in (lr.LR_FAMILY_CACHE, lr.LR_FAMILY_TREE) and p.splits == 0:
                        need = -(-((cols + 6) // 4 if cols % 4 else cols // 4) // (64 * p.waves_per_row))
                        assert p.chunks_per_lane >= need
                        assert p.chunks_per_lane in (1, 2, 3, 4, 6, 8, 12, 16, 24, 32)
                    if policy in ("ordered_fold", "fold_right"):
                        assert p.family == lr.LR_FAMILY_ORDERED and p.waves_per_row == 1
                    if policy == "ordered_tree":
                        assert p.family in (lr.LR_FAMILY_TREE, lr.LR_FAMILY_ORDERED)
                        if p.family == lr.LR_FAMILY_TREE:
                            assert cols % 4 == 0 and cols <= 32768
                    if policy == "unordered_tree":
                        assert p.family in (lr.LR_FAMILY_CACHE, lr.LR_FAMILY_STREAM, lr.LR_FAMILY_SPLIT)


def test_automatic_plan_is_legal_and_deterministic():
    for op in OPS:
        for rows, cols in [(37, 1537), (256, 3072), (64, 12289), (768, 6144), (4096, 32000), (7, 4096),
                           (1, 1), (100000, 64)]:
            for policy in POLICIES:
                al = 1 if cols % 4 == 0 else 0
                a = lr.lr_plan_for_device(F, op, rows, cols, policy, al)
                b = lr.lr_plan_for_device(F, op, rows, cols, policy, al)
                assert bytes(a) == bytes(b)
                assert lr.lr_plan_validate(F, op, rows, cols, policy, al, a) == lr.LR_OK
                assert a.family != lr.LR_FAMILY_SPLIT  # the typed calls have no workspace
                w = lr.lr_plan_for_device_ws(F, op, rows, cols, policy, al)
                assert bytes(w) == bytes(lr.lr_plan_for_device_ws(F, op, rows, cols, policy, al))
                assert lr.lr_plan_validate(F, op, rows, cols, policy, al, w) == lr.LR_OK
                if w.family != lr.LR_FAMILY_SPLIT:
                    assert bytes(w) == bytes(a)


def _plan(**kw):
    p = lr.lr_plan_for_device(F, "softmax", 768, 6144, "unordered_tree", 1)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("change", [
    dict(chunks_per_lane=5),                                 # no compiled instance
    dict(waves_per_row=1, threads_per_block=64, chunks_per_lane=6),  # stripe too small for the row
    dict(threads_per_block=512),                             # inconsistent with 64*S*Q
    dict(rows_per_block=3, threads_per_block=64 * 4 * 3, blocks=256),  # fine shape, wrong... S*Q ok
    dict(waves_per_row=17, threads_per_block=64 * 17),       # S out of range
    dict(blocks=1),                                          # wrong block count
    dict(family=lr.LR_FAMILY_ORDERED),                       # family does not match policy
    dict(vec=2),
])
def test_unrealizable_explicit_plan_is_rejected_not_clamped(change):
    p = _plan(**change)
    st = lr.lr_plan_validate(F, "softmax", 768, 6144, "unordered_tree", 1, p)
    if change.get("rows_per_block") == 3:
        # S=4, Q=3 is a legal shape: honoured exactly
        assert st == lr.LR_OK
    else:
        assert st == lr.LR_ERR_UNREALIZABLE_PLAN


def test_ordered_policy_rejects_unordered_plan():
    p = lr.lr_plan_for_device(F, "rmsnorm", 256, 3072, "unordered_tree", 1)
    assert lr.lr_plan_validate(F, "rmsnorm", 256, 3072, "ordered_fold", 1, p) == lr.LR_ERR_UNREALIZABLE_PLAN
    q = lr.lr_plan_for_device(F, "rmsnorm", 256, 3072, "ordered_fold", 1)
    assert q.family == lr.LR_FAMILY_ORDERED
    assert lr.lr_plan_validate(F, "rmsnorm", 256, 3072, "unordered_tree", 1, q) == lr.LR_ERR_UNREALIZABLE_PLAN


def test_tree_family_is_for_ordered_tree_on_aligned_rows_only():
    q = lr.lr_plan_for_device(F, "layernorm", 768, 6144, "ordered_tree", 1)
    assert q.family == lr.LR_FAMILY_TREE
    for pol in ("unordered_tree", "ordered_fold", "fold_right"):
        assert lr.lr_plan_validate(F, "layernorm", 768, 6144, pol, 1, q) == lr.LR_ERR_UNREALIZABLE_PLAN
    assert lr.lr_plan_validate(F, "layernorm", 768, 6144, "ordered_tree", 0, q) == lr.LR_ERR_UNREALIZABLE_PLAN
    # misaligned rows and rows past 128 slabs take the ordered family
    assert lr.lr_plan_for_device(F, "layernorm", 64, 12289, "ordered_tree", 0).family == lr.LR_FAMILY_ORDERED
    assert lr.lr_plan_for_device(F, "row_sum", 4, 32772, "ordered_tree", 1).family == lr.LR_FAMILY_ORDERED
    assert lr.lr_plan_for_device(F, "row_sum", 4, 32768, "ordered_tree", 1).family == lr.LR_FAMILY_TREE
    # an ordered plan serves ordered_tree too
    o = lr.lr_plan_for_device(F, "layernorm", 768, 6144, "ordered_fold", 1)
    assert lr.lr_plan_validate(F, "layernorm", 768, 6144, "ordered_tree", 1, o) == lr.LR_OK


def test_cache_plan_for_aligned_rows_does_not_cover_misaligned_rows():
    # 6144 floats over S=4 waves is exactly 6 chunks per lane when rows are
    # 16-byte aligned; a misaligned row touches one more chunk
    p = _plan(family=lr.LR_FAMILY_CACHE, waves_per_row=4, rows_per_block=1, threads_per_block=256,
              blocks=768, chunks_per_lane=6)
    assert lr.lr_plan_validate(F, "softmax", 768, 6144, "unordered_tree", 1, p) == lr.LR_OK
    assert lr.lr_plan_validate(F, "softmax", 768, 6144, "unordered_tree", 0, p) == lr.LR_ERR_UNREALIZABLE_PLAN


def test_planner_argument_errors():
    p = lr.LrPlan()
    assert lr.lib.lr_plan_for_device(ctypes.byref(F), 7, 4, 4, 0, 1, ctypes.byref(p)) == lr.LR_ERR_INVALID_ARGUMENT
    assert lr.lib.lr_plan_for_device(ctypes.byref(F), 0, 4, 4, 5, 1, ctypes.byref(p)) == lr.LR_ERR_INVALID_POLICY
    assert lr.lib.lr_plan_for_device(ctypes.byref(F), 0, 4, 0, 0, 1, ctypes.byref(p)) == lr.LR_ERR_INVALID_SHAPE
    n = ctypes.c_int32(-1)
    assert lr.lib.lr_plan_enumerate(ctypes.byref(F), 0, 4, 4, 0, 1, None, 0, ctypes.byref(n)) == lr.LR_OK
    assert n.value > 0


def _split(rows, cols, G, S, nch, aligned=1):
    p = lr.LrPlan()
    p.family, p.waves_per_row, p.rows_per_block, p.vec = lr.LR_FAMILY_SPLIT, S, 1, 4
    p.chunks_per_lane, p.threads_per_block, p.blocks, p.splits = nch, 64 * S, rows * G, G
    p.lds_bytes, p.reductions, p.row_aligned = 128, 2, aligned
    return p


def test_split_plan_legality():
    ok = _split(64, 12288, 4, 4, 3)  # 3072 chunks: 768 per segment over 256 lanes
    assert lr.lr_plan_validate(F, "layernorm", 64, 12288, "unordered_tree", 1, ok) == lr.LR_OK
    # the same stripe is one chunk short for misaligned rows (3073 chunks)
    assert lr.lr_plan_validate(F, "layernorm", 64, 12288, "unordered_tree", 0, ok) == lr.LR_ERR_UNREALIZABLE_PLAN
    bad = [
        dict(splits=1, blocks=64), dict(splits=65, blocks=64 * 65), dict(blocks=65),
        dict(chunks_per_lane=5), dict(chunks_per_lane=12), dict(chunks_per_lane=2),
        dict(rows_per_block=2, threads_per_block=512), dict(vec=1),
    ]
    for change in bad:
        p = _split(64, 12288, 4, 4, 3)
        for k, v in change.items():
            setattr(p, k, v)
        assert lr.lr_plan_validate(F, "layernorm", 64, 12288, "unordered_tree", 1, p) == \
            lr.LR_ERR_UNREALIZABLE_PLAN, change
    # no segment without a chunk of its own: splits <= the row's chunk count
    assert lr.lr_plan_validate(F, "softmax", 3, 20, "unordered_tree", 1, _split(3, 20, 5, 1, 1)) == lr.LR_OK
    assert lr.lr_plan_validate(F, "softmax", 3, 20, "unordered_tree", 1, _split(3, 20, 6, 1, 1)) == \
        lr.LR_ERR_UNREALIZABLE_PLAN
    # only the unordered policy splits rows, and other families carry no splits
    for pol in ("ordered_fold", "ordered_tree", "fold_right"):
        assert lr.lr_plan_validate(F, "layernorm", 64, 12288, pol, 1, ok) == lr.LR_ERR_UNREALIZABLE_PLAN
    c = lr.lr_plan_for_device(F, "layernorm", 64, 12288, "unordered_tree", 1)
    c.splits = 2
    assert lr.lr_plan_validate(F, "layernorm", 64, 12288, "unordered_tree", 1, c) == lr.LR_ERR_UNREALIZABLE_PLAN


def test_workspace_plan_splits_few_long_rows_only():
    for op in OPS:
        w = lr.lr_plan_for_device_ws(F, op, 64, 12288, "unordered_tree", 1)
        v = lr.lr_plan_for_device_ws(F, op, 48, 16384, "unordered_tree", 1)  # the prior: no measured entry
        if op == "add_layernorm":
            for p, rows in ((w, 64), (v, 48)):
                assert p.family == lr.LR_FAMILY_SPLIT and p.splits >= 2 and p.blocks >= 256, (op, p)
                assert lr.lr_plan_workspace_bytes(p, rows) == rows * p.splits * 8
        else:  # one launch is faster for these
            assert w.family != lr.LR_FAMILY_SPLIT and v.family != lr.LR_FAMILY_SPLIT, (op, w, v)
        # measured: one launch at 64 x 12289, with or without a workspace
        assert lr.lr_plan_for_device_ws(F, op, 64, 12289, "unordered_tree", 0).family != lr.LR_FAMILY_SPLIT
        # enough rows to fill the device, or rows too short to be worth a
        # second launch: no split
        for rows, cols in [(768, 6144), (4096, 32000), (37, 1537), (64, 512)]:
            v = lr.lr_plan_for_device_ws(F, op, rows, cols, "unordered_tree", 1 if cols % 4 == 0 else 0)
            assert v.family != lr.LR_FAMILY_SPLIT, (op, rows, cols, v)
        for pol in ("ordered_fold", "ordered_tree", "fold_right"):
            assert lr.lr_plan_for_device_ws(F, op, 64, 12289, pol, 0).family != lr.LR_FAMILY_SPLIT
    assert lr.lr_plan_workspace_bytes(None, 64) == 0


def test_split_plans_cover_each_element_once_including_empty_segments():
    # 20 floats = 5 chunks in 4 segments of 2: the last segment is empty on
    # aligned rows; misaligned rows span 6 chunks
    for rows, cols, G in [(3, 20, 4), (2, 21, 4), (5, 130, 32), (2, 12289, 4), (3, 1537, 16), (1, 4096, 64)]:
        for S in (1, 2, 3):
            aligned = 1 if cols % 4 == 0 else 0
            need = -(-(-(-((cols + 6) // 4 if not aligned else cols // 4) // G)) // (64 * S))
            nch = next(n for n in (1, 2, 3, 4, 6, 8, 99) if n >= need)
            if nch == 99:
                continue
            p = _split(rows, cols, G, S, nch, aligned)
            assert lr.lr_plan_validate(F, "softmax", rows, cols, "unordered_tree", aligned, p) == lr.LR_OK
            for ph in ((0,) if aligned else (0, 1, 2, 3)):
                assert (coverage(p, rows, cols, ph) == 1).all(), (rows, cols, G, S, ph)


def test_planner_is_thread_safe():
    """the pure planner from many host threads at once gives the plans one
    thread gives (ctypes releases the GIL during each call)"""
    import threading
    shapes = [(r, c) for r in (1, 37, 64, 256, 768, 4096) for c in (1, 257, 1537, 6144, 12289, 32000)]
    want = {(op, r, c): bytes(lr.lr_plan_for_device_ws(F, op, r, c, "unordered_tree", 0))
            for op in OPS for r, c in shapes}
    bad = []

    def worker():
        for _ in range(5):
            for (op, r, c), b in want.items():
                if bytes(lr.lr_plan_for_device_ws(F, op, r, c, "unordered_tree", 0)) != b:
                    bad.append((op, r, c))

    ts = [threading.Thread(target=worker) for _ in range(8)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not bad


def test_dispatch_rows_keep_each_dispatch_within_2_31_work_items():
    """a call runs as dispatches of lr_dispatch_rows rows: each carries at most
    2^31 work-items, pieces below the whole call hold whole workgroups of
    rows, and problems of fewer than about 2^21 rows take one dispatch"""
    limit = 1 << 31
    checked = 0
    for rows, cols in ((1, 1), (5, 3), (1 << 21, 1), ((1 << 26) + 3, 1), ((1 << 31) - 1, 1), (1 << 22, 2),
                       (3 << 20, 6144), (64, 12289), (2, (1 << 24) - 1)):
        for op in OPS:
            for policy in POLICIES:
                for aligned in ((1, 0) if cols % 4 == 0 else (0,)):
                    plans = lr.lr_plan_enumerate(F, op, rows, cols, policy, aligned)
                    plans.append(lr.lr_plan_for_device_ws(F, op, rows, cols, policy, aligned))
                    for p in plans[:: max(1, len(plans) // 10)] + plans[-1:]:
                        n = lr.lr_dispatch_rows(p, rows)
                        assert 1 <= n <= rows
                        if p.family == lr.LR_FAMILY_SPLIT:
                            blocks = n * p.splits
                        else:
                            blocks = -(-n // p.rows_per_block)
                            assert n == rows or n % p.rows_per_block == 0
                        assert blocks * p.threads_per_block <= limit, (op, rows, cols, p)
                        if rows * 64 * 16 <= limit:
                            assert n == rows
                        whole = rows * p.splits if p.family == lr.LR_FAMILY_SPLIT else -(-rows // p.rows_per_block)
                        if whole * p.threads_per_block <= limit:
                            assert n == rows  # never split without need
                        else:
                            assert (blocks + (p.splits or 1)) * p.threads_per_block > limit  # pieces are full
                        checked += 1
    assert checked > 500
    # the grid of a tall, narrow problem under a whole-wave plan does not fit
    # one dispatch; the automatic plan packs 16 rows per wave and does
    tall = (1 << 26) + 3
    whole = [p for p in lr.lr_plan_enumerate(F, "softmax", tall, 1, "unordered_tree", 0) if p.lanes_per_row == 64]
    assert whole and all(lr.lr_dispatch_rows(p, tall) < tall for p in whole)
    p = lr.lr_plan_for_device(F, "softmax", tall, 1, "unordered_tree", 0)
    assert p.lanes_per_row == 4 and lr.lr_dispatch_rows(p, tall) == tall
    assert lr.lr_dispatch_rows(None, 5) == 0 and lr.lr_dispatch_rows(p, 0) == 0


def test_prior_takes_one_lane_per_row_for_narrow_ordered_rows():
    """many rows of at most 64 floats under an ordered policy: one lane per
    row, at the smallest compiled width, aligned or not; wider rows and few
    rows keep one wave per row"""
    for cols, nch in ((1, 1), (16, 4), (32, 8), (50, 16), (64, 16)):
        for aligned in (0, 1):
            if aligned and cols % 4:
                continue
            for policy in ("ordered_fold", "ordered_tree", "fold_right"):
                p = lr.lr_plan_for_device(F, "rmsnorm", 262144, cols, policy, aligned)
                if policy == "ordered_tree" and aligned and cols >= 4:
                    continue  # narrow TREE teams take aligned rows under the tree
                assert p.lanes_per_row == 1 and p.chunks_per_lane == nch, (cols, aligned, policy, p)
    assert lr.lr_plan_for_device(F, "rmsnorm", 262144, 65, "ordered_fold", 0).lanes_per_row == 64
    assert lr.lr_plan_for_device(F, "rmsnorm", 8, 64, "ordered_fold", 1).lanes_per_row == 64
