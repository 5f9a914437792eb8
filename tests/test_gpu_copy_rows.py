"""The row copy that measures the data-movement floor (lr_copy_rows_f32)
moves every element once and nothing else, with and without the barrier
before its stores: y is bit-equal to x, including NaN payloads, the bytes
around y are untouched, and the copy works in place.
It runs under the very plans the 768 x 6144 operations launch with, and under
plans with several chunks per lane and a ragged last chunk row."""
import numpy as np
import pytest
import torch

import row_reductions_amd as lr
import synth
from gpu_util import DEV

pytestmark = pytest.mark.gpu


def plans_for(rows, cols):
    F = lr.lr_device_facts_query()
    out = [lr.lr_plan_query(op, rows, cols, "unordered_tree") for op in ("softmax", "rmsnorm", "layernorm")]
    def usable(p):
        return (p.family == lr.LR_FAMILY_CACHE and p.rows_per_block == 1 and p.lanes_per_row == 64 * p.waves_per_row
                and p.chunks_per_lane in (1, 2, 3, 4, 6, 8))
    out = [p for p in out if usable(p)]
    for p in lr.lr_plan_enumerate(F, "softmax", rows, cols, "unordered_tree", 1):
        if usable(p) and len(out) < 8:
            out.append(p)
    return out


@pytest.mark.parametrize("rows,cols", [(768, 6144), (7, 4096), (5, 1028), (3, 64)])
def test_copy_rows_bit_exact(rows, cols):
    x = synth.normal_f32(rows + cols, 0, rows * cols, 0.0, 3.0)
    bits = x.view(np.uint32)
    bits[::997] = 0x7FC00001 + (np.arange(bits[::997].size, dtype=np.uint32) & 0xFF)  # NaN payloads
    xd = torch.from_numpy(x.reshape(rows, cols)).to(DEV)
    pad = 64
    for p in plans_for(rows, cols):
        print(f"\n[gpu] copy_rows {rows}x{cols} S={p.waves_per_row} n={p.chunks_per_lane}", flush=True)
        for sync in (0, 1):
            full = torch.full((rows * cols + 2 * pad,), -7.0, device=DEV)
            y = full[pad:pad + rows * cols]
            assert lr.lr_copy_rows_f32(xd, y, rows, cols, p, sync) == lr.LR_OK
            torch.cuda.synchronize()
            got = y.cpu().numpy()
            assert (got.view(np.uint32) == bits).all(), (p, sync)
            rest = torch.cat([full[:pad], full[pad + rows * cols:]]).cpu().numpy()
            assert (rest == -7.0).all(), (p, sync)
            z = xd.clone()
            assert lr.lr_copy_rows_f32(z, z, rows, cols, p, sync) == lr.LR_OK
            torch.cuda.synchronize()
            assert (z.cpu().numpy().reshape(-1).view(np.uint32) == bits).all(), (p, sync)
