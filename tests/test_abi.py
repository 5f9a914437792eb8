"""C-ABI boundary on the CPU: the library loads, exports every function that
include/lr.h declares, and rejects bad arguments with the documented status
before making any HIP call (no GPU is needed for any check here)."""
import ctypes
import functools
import os
import re

import pytest

import row_reductions_amd as lr

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "lr.h")

# Fake, well-aligned device addresses: validation never dereferences them.
X = 0x7F0000000000
Y = 0x7F0010000000
G = 0x7F0020000000
B = 0x7F0030000000
LAB = 0x7F0040000000
LOSS = 0x7F0050000000
RES = 0x7F0060000000
SUM = 0x7F0070000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lr_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lr.lib, n), n
    assert lr.lr_version().startswith("lr ")
    for code, name in lr.STATUS.items():
        assert lr.lr_status_string(code).startswith(name)


def test_zero_rows_is_ok_without_launch():
    # succeeds with no device present: nothing is launched and no HIP call is made
    assert lr.lr_softmax_f32(X, Y, 0, 128, 0, 0) == lr.LR_OK
    assert lr.lr_rmsnorm_f32(X, None, Y, 0, 5, 1e-6, 1, 0) == lr.LR_OK
    assert lr.lr_layernorm_f32(X, None, None, Y, 0, 7, 1e-5, 0, 0) == lr.LR_OK
    assert lr.lr_cross_entropy_f32(X, LAB, LOSS, 0, 32000, 0, 0) == lr.LR_OK
    assert lr.lr_add_layernorm_f32(X, RES, None, None, Y, SUM, 0, 7, 1e-5, 0, 0) == lr.LR_OK
    assert lr.lr_row_sum_f32(X, LOSS, 0, 7, 1, 0) == lr.LR_OK
    assert lr.lr_row_minmax_f32(X, LOSS, None, 0, 7, 0, 0) == lr.LR_OK


@pytest.mark.parametrize("call,status", [
    (lambda: lr.lr_softmax_f32(None, Y, 4, 8, 0, 0), lr.LR_ERR_NULL_POINTER),
    (lambda: lr.lr_softmax_f32(X, None, 4, 8, 0, 0), lr.LR_ERR_NULL_POINTER),
    (lambda: lr.lr_cross_entropy_f32(X, None, LOSS, 4, 8, 0, 0), lr.LR_ERR_NULL_POINTER),
    (lambda: lr.lr_cross_entropy_f32(X, LAB, None, 4, 8, 0, 0), lr.LR_ERR_NULL_POINTER),
    (lambda: lr.lr_softmax_f32(X, Y, -1, 8, 0, 0), lr.LR_ERR_INVALID_SHAPE),
    (lambda: lr.lr_softmax_f32(X, Y, 4, 0, 0, 0), lr.LR_ERR_INVALID_SHAPE),
    (lambda: lr.lr_softmax_f32(X, Y, 4, -3, 0, 0), lr.LR_ERR_INVALID_SHAPE),
    (lambda: lr.lr_softmax_f32(X, Y, 4, 1 << 24, 0, 0), lr.LR_ERR_INVALID_SHAPE),
    (lambda: lr.lr_softmax_f32(X, Y, 1 << 31, 8, 0, 0), lr.LR_ERR_INVALID_SHAPE),
    (lambda: lr.lr_softmax_f32(X, Y, 4, 8, 4, 0), lr.LR_ERR_INVALID_POLICY),
    (lambda: lr.lr_softmax_f32(X, Y, 4, 8, -1, 0), lr.LR_ERR_INVALID_POLICY),
    (lambda: lr.lr_rmsnorm_f32(X, G, Y, 4, 8, float("nan"), 0, 0), lr.LR_ERR_INVALID_EPS),
    (lambda: lr.lr_rmsnorm_f32(X, G, Y, 4, 8, float("inf"), 0, 0), lr.LR_ERR_INVALID_EPS),
    (lambda: lr.lr_layernorm_f32(X, G, B, Y, 4, 8, -1e-5, 0, 0), lr.LR_ERR_INVALID_EPS),
    (lambda: lr.lr_softmax_f32(X + 2, Y, 4, 8, 0, 0), lr.LR_ERR_MISALIGNED),
    (lambda: lr.lr_rmsnorm_f32(X, G + 1, Y, 4, 8, 1e-6, 0, 0), lr.LR_ERR_MISALIGNED),
    (lambda: lr.lr_cross_entropy_f32(X, LAB + 4, LOSS, 4, 8, 0, 0), lr.LR_ERR_MISALIGNED),
    # partial overlap of input and output
    (lambda: lr.lr_softmax_f32(X, X + 4, 4, 8, 0, 0), lr.LR_ERR_ALIASING),
    (lambda: lr.lr_rmsnorm_f32(X, Y + 16, Y, 4, 8, 1e-6, 0, 0), lr.LR_ERR_ALIASING),
    (lambda: lr.lr_layernorm_f32(X, G, Y + 8, Y, 4, 8, 1e-5, 0, 0), lr.LR_ERR_ALIASING),
    (lambda: lr.lr_cross_entropy_f32(X, LAB, X + 64, 4, 8, 0, 0), lr.LR_ERR_ALIASING),
    (lambda: lr.lr_cross_entropy_f32(X, LAB, LAB + 8, 4, 8, 0, 0), lr.LR_ERR_ALIASING),
    # fused residual LayerNorm
    (lambda: lr.lr_add_layernorm_f32(X, None, G, B, Y, None, 4, 8, 1e-5, 0, 0), lr.LR_ERR_NULL_POINTER),
    (lambda: lr.lr_add_layernorm_f32(X, RES, G, B, None, SUM, 4, 8, 1e-5, 0, 0), lr.LR_ERR_NULL_POINTER),
    (lambda: lr.lr_add_layernorm_f32(X, RES, G, B, Y, SUM, 4, 8, float("nan"), 0, 0), lr.LR_ERR_INVALID_EPS),
    (lambda: lr.lr_add_layernorm_f32(X, RES + 2, G, B, Y, SUM, 4, 8, 1e-5, 0, 0), lr.LR_ERR_MISALIGNED),
    (lambda: lr.lr_add_layernorm_f32(X, RES, G, B, Y, SUM + 1, 4, 8, 1e-5, 0, 0), lr.LR_ERR_MISALIGNED),
    (lambda: lr.lr_add_layernorm_f32(X, RES, G, B, Y, SUM, 4, 8, 1e-5, 7, 0), lr.LR_ERR_INVALID_POLICY),
    (lambda: lr.lr_add_layernorm_f32(X, RES, G, B, RES + 4, None, 4, 8, 1e-5, 0, 0), lr.LR_ERR_ALIASING),
    (lambda: lr.lr_add_layernorm_f32(X, RES, G, B, Y, Y + 16, 4, 8, 1e-5, 0, 0), lr.LR_ERR_ALIASING),
    (lambda: lr.lr_add_layernorm_f32(X, RES, G, B, Y, Y, 4, 8, 1e-5, 0, 0), lr.LR_ERR_ALIASING),
    (lambda: lr.lr_add_layernorm_f32(X, RES, G, B, X, X, 4, 8, 1e-5, 0, 0), lr.LR_ERR_ALIASING),
    (lambda: lr.lr_add_layernorm_f32(X, RES, Y + 8, B, Y, SUM, 4, 8, 1e-5, 0, 0), lr.LR_ERR_ALIASING),
    (lambda: lr.lr_add_layernorm_f32(X, RES, G, SUM + 8, Y, SUM, 4, 8, 1e-5, 0, 0), lr.LR_ERR_ALIASING),
    # row sum, row minimum and maximum
    (lambda: lr.lr_row_sum_f32(X, None, 4, 8, 0, 0), lr.LR_ERR_NULL_POINTER),
    (lambda: lr.lr_row_minmax_f32(X, None, None, 4, 8, 0, 0), lr.LR_ERR_NULL_POINTER),
    (lambda: lr.lr_row_sum_f32(X, LOSS + 2, 4, 8, 0, 0), lr.LR_ERR_MISALIGNED),
    (lambda: lr.lr_row_minmax_f32(X, None, LOSS + 1, 4, 8, 0, 0), lr.LR_ERR_MISALIGNED),
    (lambda: lr.lr_row_sum_f32(X, LOSS, 4, 8, 5, 0), lr.LR_ERR_INVALID_POLICY),
    (lambda: lr.lr_add_layernorm_f32(X, RES, G, B, Y, SUM, 4, 8, 1e-5, 4, 0), lr.LR_ERR_INVALID_POLICY),
    (lambda: lr.lr_row_sum_f32(X, X + 64, 4, 8, 0, 0), lr.LR_ERR_ALIASING),
    (lambda: lr.lr_row_minmax_f32(X, LOSS, LOSS + 8, 4, 8, 0, 0), lr.LR_ERR_ALIASING),
    (lambda: lr.lr_row_minmax_f32(X, LOSS, LOSS, 4, 8, 0, 0), lr.LR_ERR_ALIASING),
    (lambda: lr.lr_row_minmax_f32(X, X, None, 4, 8, 0, 0), lr.LR_ERR_ALIASING),
    # y is x in place, but x and the residual overlap partially: rows would race
    (lambda: lr.lr_add_layernorm_f32(X, X + 16, G, B, X, None, 4, 8, 1e-5, 0, 0), lr.LR_ERR_ALIASING),
])
def test_validation_status_before_any_hip_call(call, status):
    assert call() == status


def test_with_plan_requires_plan():
    f = ctypes.POINTER(lr.LrPlan)()
    assert lr.lib.lr_softmax_f32_with_plan(X, Y, 4, 8, 0, f, 0) == lr.LR_ERR_NULL_POINTER


def test_valid_call_without_device_reports_hip_error():
    # arguments pass validation, then the device query fails on this CPU-only host
    if os.path.exists("/dev/kfd"):
        pytest.skip("a GPU is present")
    assert lr.lr_softmax_f32(X, Y, 4, 8, 0, 0) == lr.LR_ERR_HIP
    assert lr.lr_softmax_f32(X, X, 4, 8, 0, 0) == lr.LR_ERR_HIP  # in place is allowed
    for pol in (lr.LR_ORDERED_TREE, lr.LR_FOLD_RIGHT):  # every policy is accepted
        assert lr.lr_softmax_f32(X, Y, 4, 8, pol, 0) == lr.LR_ERR_HIP
    # fused residual LayerNorm: outputs may be exactly x or the residual
    assert lr.lr_add_layernorm_f32(X, RES, G, B, X, RES, 4, 8, 1e-5, 0, 0) == lr.LR_ERR_HIP
    assert lr.lr_add_layernorm_f32(X, RES, None, None, RES, X, 4, 8, 1e-5, 0, 0) == lr.LR_ERR_HIP
    assert lr.lr_add_layernorm_f32(X, X, None, None, Y, None, 4, 8, 1e-5, 0, 0) == lr.LR_ERR_HIP
    assert lr.lr_row_sum_f32(X, LOSS, 4, 8, 1, 0) == lr.LR_ERR_HIP
    assert lr.lr_row_minmax_f32(X, None, LOSS, 4, 8, 0, 0) == lr.LR_ERR_HIP


WS = 0x7F0080000000
RUN = functools.partial(lr.lr_run_f32, stream=0)  # no torch stream on a CPU host


def _split_plan(rows, cols, G=4, S=4, nch=3):
    p = lr.LrPlan()
    p.family, p.waves_per_row, p.rows_per_block, p.vec = lr.LR_FAMILY_SPLIT, S, 1, 4
    p.chunks_per_lane, p.threads_per_block, p.blocks, p.splits = nch, 64 * S, rows * G, G
    p.row_aligned = 1
    return p


@pytest.mark.parametrize("call,status", [
    (lambda: lr.lib.lr_run_f32(0, None, 4, 8, 0.0, 0, None, None, 0, None), lr.LR_ERR_NULL_POINTER),
    (lambda: RUN("softmax", 4, 8, x=X, y=Y, gamma=G), lr.LR_ERR_INVALID_ARGUMENT),
    (lambda: RUN("rmsnorm", 4, 8, 1e-6, x=X, y=Y, beta=B), lr.LR_ERR_INVALID_ARGUMENT),
    (lambda: RUN("row_sum", 4, 8, x=X, sums=LOSS, mins=SUM), lr.LR_ERR_INVALID_ARGUMENT),
    (lambda: RUN("cross_entropy", 4, 8, x=X, labels=LAB, losses=LOSS, y=Y), lr.LR_ERR_INVALID_ARGUMENT),
    (lambda: RUN(7, 4, 8, x=X, y=Y), lr.LR_ERR_INVALID_ARGUMENT),
    (lambda: RUN("softmax", 4, 8, x=X), lr.LR_ERR_NULL_POINTER),
    # workspace: NULL with a size, misaligned, overlapping a tensor of the call
    (lambda: RUN("softmax", 4, 8, workspace=0, workspace_bytes=64, x=X, y=Y), lr.LR_ERR_NULL_POINTER),
    (lambda: RUN("softmax", 4, 8, workspace=WS + 8, workspace_bytes=64, x=X, y=Y), lr.LR_ERR_MISALIGNED),
    (lambda: RUN("softmax", 4, 8, workspace=X + 64, workspace_bytes=64, x=X, y=Y), lr.LR_ERR_ALIASING),
    (lambda: RUN("layernorm", 4, 8, 1e-5, workspace=G + 16, workspace_bytes=64, x=X, y=Y, gamma=G),
     lr.LR_ERR_ALIASING),
    (lambda: RUN("cross_entropy", 4, 8, workspace=LAB - 16, workspace_bytes=32, x=X, labels=LAB,
                           losses=LOSS), lr.LR_ERR_ALIASING),
    (lambda: RUN("row_minmax", 4, 8, workspace=SUM, workspace_bytes=64, x=X, maxs=SUM + 32),
     lr.LR_ERR_ALIASING),
    # a split plan without the workspace it needs: rows * splits * 8 bytes
    (lambda: lr.lr_layernorm_f32(X, G, B, Y, 64, 12288, 1e-5, 0, plan=_split_plan(64, 12288), stream=0),
     lr.LR_ERR_WORKSPACE),
    (lambda: RUN("layernorm", 64, 12288, 1e-5, plan=_split_plan(64, 12288), workspace=WS,
                 workspace_bytes=64 * 4 * 8 - 1, x=X, y=Y), lr.LR_ERR_WORKSPACE),
    (lambda: lr.lr_row_sum_f32(X, LOSS, 64, 12288, 0, plan=_split_plan(64, 12288), stream=0), lr.LR_ERR_WORKSPACE),
    # the run call validates like the typed ones
    (lambda: RUN("rmsnorm", 4, 8, float("nan"), x=X, y=Y), lr.LR_ERR_INVALID_EPS),
    (lambda: RUN("softmax", 4, 8, policy=9, x=X, y=Y), lr.LR_ERR_INVALID_POLICY),
    (lambda: RUN("softmax", 4, 8, x=X, y=X + 4), lr.LR_ERR_ALIASING),
])
def test_run_and_workspace_validation_before_any_hip_call(call, status):
    assert call() == status


def test_run_without_device_reports_hip_error():
    if os.path.exists("/dev/kfd"):
        pytest.skip("a GPU is present")
    assert RUN("softmax", 0, 8, x=X, y=Y) == lr.LR_OK  # nothing to launch
    assert RUN("softmax", 4, 8, x=X, y=Y) == lr.LR_ERR_HIP
    ws = dict(workspace=WS, workspace_bytes=64 * 4 * 8)
    assert RUN("layernorm", 64, 12288, 1e-5, plan=_split_plan(64, 12288), x=X, y=Y, **ws) == lr.LR_ERR_HIP
    assert lr.lr_softmax_f32(X, Y, 64, 12288, stream=0, workspace=WS, workspace_bytes=1 << 20) == lr.LR_ERR_HIP
    with pytest.raises(lr.LrError):
        lr.lr_workspace_query("layernorm", 64, 12289)


def test_noalloc_refuses_an_oversized_plan_before_any_hip_call():
    # 4096 rows x 64 segments x 8 B = 2 MiB of partials > the 1 MiB array
    big = next(p for p in lr.lr_plan_enumerate(lr.lr_device_facts_mi355x(), "softmax", 4096, 1024,
                                               "unordered_tree", 1)
               if p.family == lr.LR_FAMILY_SPLIT and p.splits == 64)
    assert lr.lr_plan_workspace_bytes(big, 4096) > (1 << 20)
    assert lr.lr_run_f32_noalloc("softmax", 4096, 1024, 0.0, "unordered_tree", big, stream=0, x=X,
                                 y=Y) == lr.LR_ERR_WORKSPACE
    # the shared validation runs first, as in lr_run_f32
    assert lr.lr_run_f32_noalloc("softmax", 4, 8, 0.0, 9, stream=0, x=X, y=Y) == lr.LR_ERR_INVALID_POLICY


def test_noalloc_without_device_reports_hip_error():
    if os.path.exists("/dev/kfd"):
        pytest.skip("a GPU is present")
    assert lr.lr_run_f32_noalloc("layernorm", 64, 12288, 1e-5, "unordered_tree", _split_plan(64, 12288),
                                 stream=0, x=X, y=Y) == lr.LR_ERR_HIP


def test_copy_rows_validates_before_any_hip_call():
    F = lr.lr_device_facts_mi355x()
    p = lr.lr_plan_for_device(F, "rmsnorm", 768, 6144, "unordered_tree", 1)
    assert p.family == lr.LR_FAMILY_CACHE and p.rows_per_block == 1
    assert lr.lr_copy_rows_f32(X, Y, 0, 6144, p, 1, 0) == lr.LR_OK  # nothing to launch
    assert lr.lib.lr_copy_rows_f32(X, Y, 4, 6144, None, 1, 0) == lr.LR_ERR_NULL_POINTER
    assert lr.lr_copy_rows_f32(X, Y, 4, 6144, p, 2, 0) == lr.LR_ERR_INVALID_ARGUMENT
    assert lr.lr_copy_rows_f32(None, Y, 4, 6144, p, 1, 0) == lr.LR_ERR_NULL_POINTER
    assert lr.lr_copy_rows_f32(X, Y, -1, 6144, p, 1, 0) == lr.LR_ERR_INVALID_SHAPE
    assert lr.lr_copy_rows_f32(X, Y, 4, 6142, p, 1, 0) == lr.LR_ERR_MISALIGNED
    assert lr.lr_copy_rows_f32(X + 4, Y, 4, 6144, p, 1, 0) == lr.LR_ERR_MISALIGNED
    assert lr.lr_copy_rows_f32(X, X + 16, 4, 6144, p, 1, 0) == lr.LR_ERR_ALIASING
    # lanes that do not cover the row
    assert lr.lr_copy_rows_f32(X, Y, 4, 64 * p.waves_per_row * p.chunks_per_lane * 4 + 4, p, 1, 0) \
        == lr.LR_ERR_UNREALIZABLE_PLAN
    # not a one-row CACHE plan, or a chunk count with no compiled copy
    st = next(q for q in lr.lr_plan_enumerate(F, "rmsnorm", 768, 6144, "unordered_tree", 1)
              if q.family == lr.LR_FAMILY_STREAM)
    assert lr.lr_copy_rows_f32(X, Y, 4, 6144, st, 1, 0) == lr.LR_ERR_UNREALIZABLE_PLAN
    packed = next(q for q in lr.lr_plan_enumerate(F, "softmax", 768, 256, "unordered_tree", 1)
                  if q.family == lr.LR_FAMILY_CACHE and q.rows_per_block > 1)
    assert lr.lr_copy_rows_f32(X, Y, 4, 256, packed, 1, 0) == lr.LR_ERR_UNREALIZABLE_PLAN
    big = next(q for q in lr.lr_plan_enumerate(F, "softmax", 4, 32768, "unordered_tree", 1)
               if q.family == lr.LR_FAMILY_CACHE and q.chunks_per_lane == 16)
    assert lr.lr_copy_rows_f32(X, Y, 4, 32768, big, 1, 0) == lr.LR_ERR_UNREALIZABLE_PLAN


def test_device_memory_query_checks_its_outputs():
    import ctypes
    v = ctypes.c_int32(0)
    assert lr.lib.lr_device_memory_query(None, ctypes.byref(v)) == lr.LR_ERR_NULL_POINTER
    assert lr.lib.lr_device_memory_query(ctypes.byref(v), None) == lr.LR_ERR_NULL_POINTER
    if os.path.exists("/dev/kfd"):
        pytest.skip("a GPU is present")
    with pytest.raises(lr.LrError):
        lr.lr_device_memory_query()
