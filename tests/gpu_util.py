"""Helpers for the GPU tests: device buffers, running an op through the C ABI,
and the parity bar |gpu - ref| <= 1e-6 + 1e-5 |ref|."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import row_reductions_amd as lr

ATOL = 1e-6
RTOL = 1e-5
DEV = "cuda:0"


def dev(a: np.ndarray | None, pad: int = 0):
    """Copy to the GPU.  With pad > 0 the data sits `pad` elements into a
    larger buffer (returns (view, full_buffer))."""
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if pad == 0:
        return t.to(DEV)
    flat = t.reshape(-1)
    full = torch.empty(flat.numel() + 2 * pad + 8, dtype=t.dtype, device=DEV)
    view = full[pad:pad + flat.numel()]
    view.copy_(flat.to(DEV))
    return view.view(t.shape), full


def workspace_for(plan, rows):
    """A workspace for a split-family plan (None for any other), filled with
    NaN bytes: the call must overwrite every partial it reads."""
    n = lr.lr_plan_workspace_bytes(plan, rows) if plan is not None else 0
    if n == 0:
        return None
    return torch.full((n,), 0xFF, dtype=torch.uint8, device=DEV)


def run_gpu(op: str, inp: dict, eps=None, policy="unordered_tree", plan=None, x_pad=0, y_pad=0,
            canary=None, in_place=False, workspace=None):
    """Runs `op` on the GPU and returns (output as numpy, status, extras).
    A split-family plan gets a workspace of its own unless one is given."""
    x = inp["logits"] if op == "cross_entropy" else inp["x"]
    rows, cols = x.shape
    xv = dev(x, x_pad)[0] if x_pad else dev(x)
    extras = {}
    ws = workspace if workspace is not None else workspace_for(plan, rows)
    if op == "cross_entropy":
        lab = dev(inp["labels"])
        out = torch.empty(rows, dtype=torch.float32, device=DEV)
        st = lr.lr_cross_entropy_f32(xv, lab, out, rows, cols, policy, plan=plan, workspace=ws)
    else:
        if in_place:
            yv, yfull = xv, None
        elif y_pad:
            yfull = torch.empty(rows * cols + 2 * y_pad + 8, dtype=torch.float32, device=DEV)
            if canary is not None:
                yfull.fill_(canary)
            yv = yfull[y_pad:y_pad + rows * cols].view(rows, cols)
        else:
            yfull = None
            yv = torch.empty(rows, cols, dtype=torch.float32, device=DEV)
        if op == "softmax":
            st = lr.lr_softmax_f32(xv, yv, rows, cols, policy, plan=plan, workspace=ws)
        elif op == "rmsnorm":
            st = lr.lr_rmsnorm_f32(xv, dev(inp.get("gamma")), yv, rows, cols, eps, policy, plan=plan, workspace=ws)
        else:
            st = lr.lr_layernorm_f32(xv, dev(inp.get("gamma")), dev(inp.get("beta")), yv, rows, cols, eps,
                                     policy, plan=plan, workspace=ws)
        out = yv
        extras["yfull"] = yfull
    torch.cuda.synchronize()
    res = out.cpu().numpy()
    if extras.get("yfull") is not None:
        extras["yfull"] = extras["yfull"].cpu().numpy()
    return res, st, extras


def within_bar(got: np.ndarray, ref: np.ndarray):
    err = np.abs(got.astype(np.float64) - ref)
    bound = ATOL + RTOL * np.abs(ref)
    ok = err <= bound
    return bool(ok.all()), float((err / bound).max()) if err.size else 0.0


def assert_parity(got, ref, what=""):
    ok, worst = within_bar(got, ref)
    if not ok:
        err = np.abs(got.astype(np.float64) - ref)
        i = np.unravel_index(np.argmax(err - (ATOL + RTOL * np.abs(ref))), ref.shape)
        raise AssertionError(f"{what}: parity fails at {i}: gpu={got[i]!r} ref={ref[i]!r} "
                             f"(worst err/bound {worst:.3g})")
    return worst


def ref_of(op: str, inp: dict, eps=None):
    return oracle.run(op, inp, eps)


U32 = 2.0 ** -24


def gamma_n(n: int) -> float:
    """Higham's gamma_n = n u / (1 - n u), u = 2^-24: the relative error bound
    of a serial FP32 sum of n nonnegative terms (n - 1 roundings)."""
    return n * U32 / (1.0 - n * U32)


def check_output(op: str, inp: dict, eps, policy: str, got: np.ndarray, what: str = ""):
    """The parity gate for one GPU result.

    unordered_tree: |gpu - ref| <= 1e-6 + 1e-5 |ref| against the double oracle.
    ordered_fold:   RMSNorm / LayerNorm must equal the CPU FP32 left-fold replay
                    bit for bit (their FP32 result is unique); softmax and
                    cross-entropy (whose exp/log are the device's own) must lie
                    within the bar widened by the serial-sum bound
                    gamma_{cols-1} of their sum of exponentials."""
    what = f"{what} [{policy}]"
    if policy != "ordered_fold":
        return assert_parity(got, ref_of(op, inp, eps), what)
    if op == "rmsnorm":
        rep = oracle.rmsnorm_fold_f32(inp["x"], inp.get("gamma"), eps)
    elif op == "layernorm":
        rep = oracle.layernorm_fold_f32(inp["x"], inp.get("gamma"), inp.get("beta"), eps)
    else:
        x = inp["logits"] if op == "cross_entropy" else inp["x"]
        g = gamma_n(x.shape[1] - 1)
        ref = ref_of(op, inp, eps)
        err = np.abs(got.astype(np.float64) - ref)
        bound = ATOL + (RTOL + g) * np.abs(ref) + (g if op == "cross_entropy" else 0.0)
        if not (err <= bound).all():
            i = np.unravel_index(np.argmax(err - bound), ref.shape)
            raise AssertionError(f"{what}: outside the ordered-fold bound at {i}: gpu={got[i]!r} ref={ref[i]!r}")
        return float((err / bound).max())
    if not np.array_equal(got.view(np.uint32), rep.view(np.uint32)):
        bad = np.argwhere(got.view(np.uint32) != rep.view(np.uint32))[0]
        raise AssertionError(f"{what}: differs from the FP32 replay at {tuple(bad)}: "
                             f"gpu={got[tuple(bad)]!r} replay={rep[tuple(bad)]!r}")
    return 0.0


GUARD = 16                  # floats of guard on each side of a placed tensor
CANARY = -1.5 * 2.0 ** 126  # guard value (exact in FP32)


def placed(a, off):
    """`a` (float32) on the device `off` floats past a 16-byte boundary,
    between guard regions of CANARY: (view, whole buffer)."""
    flat = np.ascontiguousarray(a, dtype=np.float32).reshape(-1)
    full = torch.full((flat.size + 2 * GUARD + off,), CANARY, dtype=torch.float32, device=DEV)
    view = full[GUARD + off:GUARD + off + flat.size]
    view.copy_(torch.from_numpy(flat).to(DEV))
    return view.view(a.shape), full


def guards_intact(view, full):
    f = full.cpu().numpy()
    start = view.storage_offset() - full.storage_offset()
    return bool((f[:start] == CANARY).all() and (f[start + view.numel():] == CANARY).all())


def bits_equal(got, rep, what):
    if not np.array_equal(got.view(np.uint32), rep.view(np.uint32)):
        bad = tuple(np.argwhere(got.view(np.uint32) != rep.view(np.uint32))[0])
        raise AssertionError(f"{what}: differs from the FP32 replay at {bad}: {got[bad]!r} vs {rep[bad]!r}")
