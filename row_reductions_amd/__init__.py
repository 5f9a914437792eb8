"""Python binding of liblr.so, the MI355X FP32 row-reduction library.

Argument marshalling only: every entry point forwards its arguments to the
C function of the same name (declared in include/lr.h) and returns its
``lr_status`` code.  All computation happens in the HIP kernels.  Tensor
arguments may be torch tensors (their ``data_ptr()`` is passed), plain
integer device addresses, or None for optional pointers; ``stream`` may be a
torch stream, an integer ``hipStream_t`` handle, or None for the current
torch stream.

Importing this package raises ImportError when liblr.so has not been built
(``python row_reductions_amd/build.py``): there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblr.so")

# lr_reduction_policy
LR_UNORDERED_TREE = 0
LR_ORDERED_FOLD = 1  # fold_left
LR_ORDERED_TREE = 2
LR_FOLD_RIGHT = 3
LR_FOLD_LEFT = LR_ORDERED_FOLD
POLICIES = {"unordered_tree": LR_UNORDERED_TREE, "ordered_fold": LR_ORDERED_FOLD, "fold_left": LR_FOLD_LEFT,
            "ordered_tree": LR_ORDERED_TREE, "fold_right": LR_FOLD_RIGHT}

# lr_op
LR_OP_SOFTMAX, LR_OP_RMSNORM, LR_OP_LAYERNORM, LR_OP_CROSS_ENTROPY = 0, 1, 2, 3
LR_OP_ADD_LAYERNORM, LR_OP_ROW_SUM, LR_OP_ROW_MINMAX = 4, 5, 6
OPS = {"softmax": LR_OP_SOFTMAX, "rmsnorm": LR_OP_RMSNORM, "layernorm": LR_OP_LAYERNORM,
       "cross_entropy": LR_OP_CROSS_ENTROPY, "add_layernorm": LR_OP_ADD_LAYERNORM,
       "row_sum": LR_OP_ROW_SUM, "row_minmax": LR_OP_ROW_MINMAX}

# lr_family
LR_FAMILY_CACHE, LR_FAMILY_STREAM, LR_FAMILY_ORDERED, LR_FAMILY_TREE, LR_FAMILY_SPLIT = 0, 1, 2, 3, 4
FAMILY_NAMES = {0: "cache", 1: "stream", 2: "ordered", 3: "tree", 4: "split"}

# lr_status
STATUS = {
    0: "LR_OK", 1: "LR_ERR_NULL_POINTER", 2: "LR_ERR_INVALID_SHAPE", 3: "LR_ERR_INVALID_EPS",
    4: "LR_ERR_INVALID_POLICY", 5: "LR_ERR_MISALIGNED", 6: "LR_ERR_ALIASING",
    7: "LR_ERR_UNREALIZABLE_PLAN", 8: "LR_ERR_HIP", 9: "LR_ERR_INVALID_ARGUMENT", 10: "LR_ERR_WORKSPACE",
}
LR_OK = 0
globals().update({v: k for k, v in STATUS.items()})


class LrPlan(ctypes.Structure):
    _fields_ = [
        ("family", ctypes.c_int32),
        ("waves_per_row", ctypes.c_int32),
        ("rows_per_block", ctypes.c_int32),
        ("vec", ctypes.c_int32),
        ("chunks_per_lane", ctypes.c_int32),
        ("threads_per_block", ctypes.c_int32),
        ("blocks", ctypes.c_int64),
        ("lds_bytes", ctypes.c_int32),
        ("reductions", ctypes.c_int32),
        ("row_aligned", ctypes.c_int32),
        ("splits", ctypes.c_int32),
        ("lanes_per_row", ctypes.c_int32),
    ]

    def as_dict(self) -> dict:
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["family"] = FAMILY_NAMES.get(self.family, self.family)
        return d

    def __repr__(self) -> str:
        return "LrPlan(%s)" % ", ".join("%s=%s" % kv for kv in self.as_dict().items())


TENSOR_FIELDS = ("x", "residual", "gamma", "beta", "labels", "y", "sum_out", "losses", "sums", "mins", "maxs")


class LrTensors(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in TENSOR_FIELDS]


class LrDeviceFacts(ctypes.Structure):
    _fields_ = [
        ("compute_units", ctypes.c_int32),
        ("max_threads_per_block", ctypes.c_int32),
        ("simds_per_cu", ctypes.c_int32),
        ("wave_size", ctypes.c_int32),
    ]


class LrError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}" if what else STATUS.get(status, str(status)))


def _load():
    # torch bundles its own HIP runtime (soname libamdhip64.so.7).  Loading
    # torch first makes liblr.so bind to that same runtime, so device
    # pointers and stream handles from torch are valid in the library; loaded
    # the other way round the process would hold two HIP runtimes.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python row_reductions_amd/build.py` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    PP = ctypes.POINTER(LrPlan)
    PF = ctypes.POINTER(LrDeviceFacts)
    sigs = {
        "lr_softmax_f32": [P, P, I64, I64, I32, P],
        "lr_rmsnorm_f32": [P, P, P, I64, I64, F32, I32, P],
        "lr_layernorm_f32": [P, P, P, P, I64, I64, F32, I32, P],
        "lr_cross_entropy_f32": [P, P, P, I64, I64, I32, P],
        "lr_add_layernorm_f32": [P, P, P, P, P, P, I64, I64, F32, I32, P],
        "lr_row_sum_f32": [P, P, I64, I64, I32, P],
        "lr_row_minmax_f32": [P, P, P, I64, I64, I32, P],
        "lr_copy_rows_f32": [P, P, I64, I64, PP, I32, P],
        "lr_softmax_f32_with_plan": [P, P, I64, I64, I32, PP, P],
        "lr_rmsnorm_f32_with_plan": [P, P, P, I64, I64, F32, I32, PP, P],
        "lr_layernorm_f32_with_plan": [P, P, P, P, I64, I64, F32, I32, PP, P],
        "lr_cross_entropy_f32_with_plan": [P, P, P, I64, I64, I32, PP, P],
        "lr_add_layernorm_f32_with_plan": [P, P, P, P, P, P, I64, I64, F32, I32, PP, P],
        "lr_row_sum_f32_with_plan": [P, P, I64, I64, I32, PP, P],
        "lr_row_minmax_f32_with_plan": [P, P, P, I64, I64, I32, PP, P],
        "lr_device_facts_query": [PF],
        "lr_device_memory_query": [ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)],
        "lr_plan_query": [I32, I64, I64, I32, PP],
        "lr_plan_for_device": [PF, I32, I64, I64, I32, I32, PP],
        "lr_plan_enumerate": [PF, I32, I64, I64, I32, I32, PP, I32, ctypes.POINTER(I32)],
        "lr_plan_validate": [PF, I32, I64, I64, I32, I32, PP],
        "lr_coverage_check": [PP, I64, I64, I32, P],
        "lr_run_f32": [I32, ctypes.POINTER(LrTensors), I64, I64, F32, I32, PP, P, ctypes.c_uint64, P],
        "lr_run_f32_noalloc": [I32, ctypes.POINTER(LrTensors), I64, I64, F32, I32, PP, P],
        "lr_workspace_query": [I32, I64, I64, I32, ctypes.POINTER(ctypes.c_uint64)],
        "lr_plan_for_device_ws": [PF, I32, I64, I64, I32, I32, PP],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.lr_plan_workspace_bytes.argtypes = [PP, I64]
    lib.lr_plan_workspace_bytes.restype = ctypes.c_uint64
    lib.lr_dispatch_rows.argtypes = [PP, I64]
    lib.lr_dispatch_rows.restype = I64
    lib.lr_device_facts_mi355x.argtypes = [PF]
    lib.lr_device_facts_mi355x.restype = None
    lib.lr_status_string.argtypes = [ctypes.c_int]
    lib.lr_status_string.restype = ctypes.c_char_p
    lib.lr_version.argtypes = []
    lib.lr_version.restype = ctypes.c_char_p
    return lib


lib = _load()

# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _policy(p):
    return POLICIES[p] if isinstance(p, str) else int(p)


def _op(o):
    return OPS[o] if isinstance(o, str) else int(o)


def _nbytes(t, n):
    if n is not None:
        return int(n)
    if t is None:
        return 0
    return t.numel() * t.element_size()


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI); each returns the lr_status code
# ---------------------------------------------------------------------------


def lr_run_f32(op, rows, cols, eps=0.0, policy=LR_UNORDERED_TREE, plan=None, workspace=None,
               workspace_bytes=None, stream=None, **tensors) -> int:
    """lr_run_f32: ``tensors`` are the lr_tensors members by name (x, y,
    gamma, ...).  ``workspace`` is a device tensor or address;
    ``workspace_bytes`` defaults to the tensor's size."""
    unknown = set(tensors) - set(TENSOR_FIELDS)
    if unknown:
        raise TypeError("unknown tensor arguments: %s" % sorted(unknown))
    t = LrTensors(**{k: _ptr(v) for k, v in tensors.items()})
    if workspace is not None and workspace_bytes is None and isinstance(workspace, int):
        raise TypeError("workspace_bytes is required with a raw workspace address")
    return lib.lr_run_f32(_op(op), ctypes.byref(t), rows, cols, eps, _policy(policy),
                          None if plan is None else ctypes.byref(plan), _ptr(workspace),
                          _nbytes(workspace, workspace_bytes), _stream(stream))


def lr_run_f32_noalloc(op, rows, cols, eps=0.0, policy=LR_UNORDERED_TREE, plan=None, stream=None, **tensors) -> int:
    """lr_run_f32_noalloc: lr_run_f32 with the library's own device array in
    place of a workspace (LR_NOALLOC_SCRATCH_BYTES bytes per GPU)."""
    unknown = set(tensors) - set(TENSOR_FIELDS)
    if unknown:
        raise TypeError("unknown tensor arguments: %s" % sorted(unknown))
    t = LrTensors(**{k: _ptr(v) for k, v in tensors.items()})
    return lib.lr_run_f32_noalloc(_op(op), ctypes.byref(t), rows, cols, eps, _policy(policy),
                                  None if plan is None else ctypes.byref(plan), _stream(stream))


def lr_workspace_query(op, rows, cols, policy=LR_UNORDERED_TREE) -> int:
    n = ctypes.c_uint64(0)
    st = lib.lr_workspace_query(_op(op), rows, cols, _policy(policy), ctypes.byref(n))
    if st != LR_OK:
        raise LrError(st, "lr_workspace_query")
    return n.value


def lr_plan_workspace_bytes(plan, rows) -> int:
    return int(lib.lr_plan_workspace_bytes(None if plan is None else ctypes.byref(plan), rows))


def lr_dispatch_rows(plan, rows) -> int:
    return int(lib.lr_dispatch_rows(None if plan is None else ctypes.byref(plan), rows))


def lr_softmax_f32(x, y, rows, cols, policy=LR_UNORDERED_TREE, stream=None, plan=None, workspace=None,
                   workspace_bytes=None) -> int:
    if workspace is not None:
        return lr_run_f32("softmax", rows, cols, 0.0, policy, plan, workspace, workspace_bytes, stream, x=x, y=y)
    if plan is None:
        return lib.lr_softmax_f32(_ptr(x), _ptr(y), rows, cols, _policy(policy), _stream(stream))
    return lib.lr_softmax_f32_with_plan(_ptr(x), _ptr(y), rows, cols, _policy(policy),
                                        ctypes.byref(plan), _stream(stream))


def lr_rmsnorm_f32(x, gamma, y, rows, cols, eps, policy=LR_UNORDERED_TREE, stream=None, plan=None,
                   workspace=None, workspace_bytes=None) -> int:
    if workspace is not None:
        return lr_run_f32("rmsnorm", rows, cols, eps, policy, plan, workspace, workspace_bytes, stream,
                          x=x, gamma=gamma, y=y)
    if plan is None:
        return lib.lr_rmsnorm_f32(_ptr(x), _ptr(gamma), _ptr(y), rows, cols, eps, _policy(policy),
                                  _stream(stream))
    return lib.lr_rmsnorm_f32_with_plan(_ptr(x), _ptr(gamma), _ptr(y), rows, cols, eps, _policy(policy),
                                        ctypes.byref(plan), _stream(stream))


def lr_layernorm_f32(x, gamma, beta, y, rows, cols, eps, policy=LR_UNORDERED_TREE, stream=None, plan=None,
                     workspace=None, workspace_bytes=None) -> int:
    if workspace is not None:
        return lr_run_f32("layernorm", rows, cols, eps, policy, plan, workspace, workspace_bytes, stream,
                          x=x, gamma=gamma, beta=beta, y=y)
    if plan is None:
        return lib.lr_layernorm_f32(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), rows, cols, eps,
                                    _policy(policy), _stream(stream))
    return lib.lr_layernorm_f32_with_plan(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), rows, cols, eps,
                                          _policy(policy), ctypes.byref(plan), _stream(stream))


def lr_cross_entropy_f32(logits, labels, losses, rows, cols, policy=LR_UNORDERED_TREE, stream=None, plan=None,
                         workspace=None, workspace_bytes=None) -> int:
    if workspace is not None:
        return lr_run_f32("cross_entropy", rows, cols, 0.0, policy, plan, workspace, workspace_bytes, stream,
                          x=logits, labels=labels, losses=losses)
    if plan is None:
        return lib.lr_cross_entropy_f32(_ptr(logits), _ptr(labels), _ptr(losses), rows, cols,
                                        _policy(policy), _stream(stream))
    return lib.lr_cross_entropy_f32_with_plan(_ptr(logits), _ptr(labels), _ptr(losses), rows, cols,
                                              _policy(policy), ctypes.byref(plan), _stream(stream))


def lr_add_layernorm_f32(x, residual, gamma, beta, y, sum_out, rows, cols, eps, policy=LR_UNORDERED_TREE,
                         stream=None, plan=None, workspace=None, workspace_bytes=None) -> int:
    if workspace is not None:
        return lr_run_f32("add_layernorm", rows, cols, eps, policy, plan, workspace, workspace_bytes, stream,
                          x=x, residual=residual, gamma=gamma, beta=beta, y=y, sum_out=sum_out)
    if plan is None:
        return lib.lr_add_layernorm_f32(_ptr(x), _ptr(residual), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(sum_out),
                                        rows, cols, eps, _policy(policy), _stream(stream))
    return lib.lr_add_layernorm_f32_with_plan(_ptr(x), _ptr(residual), _ptr(gamma), _ptr(beta), _ptr(y),
                                              _ptr(sum_out), rows, cols, eps, _policy(policy),
                                              ctypes.byref(plan), _stream(stream))


def lr_copy_rows_f32(x, y, rows, cols, plan, sync=1, stream=None) -> int:
    """Row copy through the CACHE family's load/store path (a floor measurement)."""
    return lib.lr_copy_rows_f32(_ptr(x), _ptr(y), rows, cols, ctypes.byref(plan), sync, _stream(stream))


def lr_row_sum_f32(x, sums, rows, cols, policy=LR_UNORDERED_TREE, stream=None, plan=None, workspace=None,
                   workspace_bytes=None) -> int:
    if workspace is not None:
        return lr_run_f32("row_sum", rows, cols, 0.0, policy, plan, workspace, workspace_bytes, stream,
                          x=x, sums=sums)
    if plan is None:
        return lib.lr_row_sum_f32(_ptr(x), _ptr(sums), rows, cols, _policy(policy), _stream(stream))
    return lib.lr_row_sum_f32_with_plan(_ptr(x), _ptr(sums), rows, cols, _policy(policy), ctypes.byref(plan),
                                        _stream(stream))


def lr_row_minmax_f32(x, mins, maxs, rows, cols, policy=LR_UNORDERED_TREE, stream=None, plan=None,
                      workspace=None, workspace_bytes=None) -> int:
    if workspace is not None:
        return lr_run_f32("row_minmax", rows, cols, 0.0, policy, plan, workspace, workspace_bytes, stream,
                          x=x, mins=mins, maxs=maxs)
    if plan is None:
        return lib.lr_row_minmax_f32(_ptr(x), _ptr(mins), _ptr(maxs), rows, cols, _policy(policy),
                                     _stream(stream))
    return lib.lr_row_minmax_f32_with_plan(_ptr(x), _ptr(mins), _ptr(maxs), rows, cols, _policy(policy),
                                           ctypes.byref(plan), _stream(stream))


def lr_device_facts_mi355x() -> LrDeviceFacts:
    f = LrDeviceFacts()
    lib.lr_device_facts_mi355x(ctypes.byref(f))
    return f


def lr_device_facts_query() -> LrDeviceFacts:
    f = LrDeviceFacts()
    st = lib.lr_device_facts_query(ctypes.byref(f))
    if st != LR_OK:
        raise LrError(st, "lr_device_facts_query")
    return f


def lr_device_memory_query() -> tuple:
    """(memory clock in kHz, memory bus width in bits) of the current device."""
    clk, bus = ctypes.c_int32(0), ctypes.c_int32(0)
    st = lib.lr_device_memory_query(ctypes.byref(clk), ctypes.byref(bus))
    if st != LR_OK:
        raise LrError(st, "lr_device_memory_query")
    return clk.value, bus.value


def lr_plan_query(op, rows, cols, policy=LR_UNORDERED_TREE) -> LrPlan:
    p = LrPlan()
    st = lib.lr_plan_query(_op(op), rows, cols, _policy(policy), ctypes.byref(p))
    if st != LR_OK:
        raise LrError(st, "lr_plan_query")
    return p


def lr_plan_for_device(facts, op, rows, cols, policy=LR_UNORDERED_TREE, row_aligned=1) -> LrPlan:
    p = LrPlan()
    st = lib.lr_plan_for_device(ctypes.byref(facts), _op(op), rows, cols, _policy(policy), row_aligned,
                                ctypes.byref(p))
    if st != LR_OK:
        raise LrError(st, "lr_plan_for_device")
    return p


def lr_plan_for_device_ws(facts, op, rows, cols, policy=LR_UNORDERED_TREE, row_aligned=1) -> LrPlan:
    p = LrPlan()
    st = lib.lr_plan_for_device_ws(ctypes.byref(facts), _op(op), rows, cols, _policy(policy), row_aligned,
                                   ctypes.byref(p))
    if st != LR_OK:
        raise LrError(st, "lr_plan_for_device_ws")
    return p


def lr_plan_enumerate(facts, op, rows, cols, policy=LR_UNORDERED_TREE, row_aligned=1) -> list:
    n = ctypes.c_int32(0)
    st = lib.lr_plan_enumerate(ctypes.byref(facts), _op(op), rows, cols, _policy(policy), row_aligned,
                               None, 0, ctypes.byref(n))
    if st != LR_OK:
        raise LrError(st, "lr_plan_enumerate")
    arr = (LrPlan * max(1, n.value))()
    st = lib.lr_plan_enumerate(ctypes.byref(facts), _op(op), rows, cols, _policy(policy), row_aligned,
                               arr, n.value, ctypes.byref(n))
    if st != LR_OK:
        raise LrError(st, "lr_plan_enumerate")
    return [arr[i] for i in range(n.value)]


def lr_plan_validate(facts, op, rows, cols, policy, row_aligned, plan) -> int:
    return lib.lr_plan_validate(ctypes.byref(facts), _op(op), rows, cols, _policy(policy), row_aligned,
                                ctypes.byref(plan))


def lr_coverage_check(plan, rows, cols, phase, counts_ptr) -> int:
    return lib.lr_coverage_check(ctypes.byref(plan), rows, cols, phase, counts_ptr)


def lr_status_string(status: int) -> str:
    return lib.lr_status_string(status).decode()


def lr_version() -> str:
    return lib.lr_version().decode()


def check(status: int, what: str = "") -> None:
    """Raise LrError unless status is LR_OK."""
    if status != LR_OK:
        raise LrError(status, what)
