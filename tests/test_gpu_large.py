"""Tensors of more than 2^31 elements: every row offset is 64-bit in the
kernels (row * cols), and this checks it on tensors that cross the 2^31
element (8 GiB) boundary, in the CACHE, STREAM and TREE families and on a
misaligned row length.  Inputs are generated on the device from a fixed seed
(torch.randn) -- at 8.6 GB per tensor the host generator would dominate the
run -- and sampled rows, including the ones on both sides of the boundary and
the last row, are copied back and checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import row_reductions_amd as lr
from gpu_util import DEV, assert_parity

pytestmark = pytest.mark.gpu

BOUNDARY = 2 ** 31


def sample_rows(rows, cols):
    b = BOUNDARY // cols  # the row that holds element 2^31
    return sorted({0, 1, b - 1, b, b + 1, rows // 2, rows - 2, rows - 1})


@pytest.mark.parametrize("op,cols,policy", [
    ("softmax", 32768, "unordered_tree"),       # CACHE, aligned
    ("layernorm", 32769, "unordered_tree"),     # misaligned rows (STREAM at this length)
    ("softmax", 40000, "unordered_tree"),       # STREAM
    ("rmsnorm", 32768, "ordered_tree"),         # TREE
    ("cross_entropy", 32768, "unordered_tree"),
    ("row_sum", 32768, "unordered_tree"),
])
def test_tensor_past_two_to_the_31(op, cols, policy):
    rows = BOUNDARY // cols + 64
    assert rows * cols > BOUNDARY
    print(f"\n[gpu] large {op} {rows}x{cols} {policy} ({rows * cols * 4 / 2**30:.1f} GiB)", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(11)
    x = torch.randn(rows, cols, device=DEV, generator=gen)
    idx = sample_rows(rows, cols)
    g = torch.rand(cols, device=DEV, generator=gen) + 0.5
    b = torch.randn(cols, device=DEV, generator=gen) * 0.1
    if op in ("cross_entropy", "row_sum"):
        out = torch.empty(rows, device=DEV)
        if op == "cross_entropy":
            lab = torch.randint(0, cols, (rows,), device=DEV, generator=gen)
            lr.check(lr.lr_cross_entropy_f32(x, lab, out, rows, cols, policy))
        else:
            lr.check(lr.lr_row_sum_f32(x, out, rows, cols, policy))
        torch.cuda.synchronize()
        xs = x[idx].cpu().numpy()
        got = out[idx].cpu().numpy()
        if op == "cross_entropy":
            ref = oracle.cross_entropy(xs, lab[idx].cpu().numpy())
            assert_parity(got, ref, op)
        else:
            ref = oracle.row_sum(xs)
            bound = 1e-6 + 1e-5 * np.abs(xs.astype(np.float64)).sum(axis=1)
            assert (np.abs(got - ref) <= bound).all()
        return
    y = torch.empty_like(x)
    if op == "softmax":
        lr.check(lr.lr_softmax_f32(x, y, rows, cols, policy))
    elif op == "rmsnorm":
        lr.check(lr.lr_rmsnorm_f32(x, g, y, rows, cols, 1e-6, policy))
    else:
        lr.check(lr.lr_layernorm_f32(x, g, b, y, rows, cols, 1e-5, policy))
    torch.cuda.synchronize()
    xs = x[idx].cpu().numpy()
    got = y[idx].cpu().numpy()
    gh, bh = g.cpu().numpy(), b.cpu().numpy()
    if op == "softmax":
        assert_parity(got, oracle.softmax(xs), op)
    elif op == "rmsnorm":
        rep = oracle.rmsnorm_ordered_f32(xs, gh, 1e-6, policy)
        assert np.array_equal(got.view(np.uint32), rep.view(np.uint32))
    else:
        assert_parity(got, oracle.layernorm(xs, gh, bh, 1e-5), op)
    del x, y
    torch.cuda.empty_cache()
