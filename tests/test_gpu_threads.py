"""Thread safety of the C ABI on the GPU: host threads, each with its own
stream (default priority), buffers and split-row workspace, call the
library at the same time (ctypes releases the GIL during each call).  Every
result must equal, bit for bit, the same call made alone on one thread: a
fixed plan is repeatable, and no call may see another's arguments or
workspace."""
import threading

import numpy as np
import pytest
import torch

import row_reductions_amd as lr
import synth
from gpu_util import DEV

pytestmark = pytest.mark.gpu

THREADS = 6
ITERS = 25


def make_case(k):
    """Inputs for thread k: softmax 37x1537, LayerNorm 64x12289 (split through
    a workspace), cross-entropy 256x3072 and RMSNorm 768x6144."""
    s = torch.from_numpy(synth.softmax_inputs(37, 1537, seed=k, std=4.0)["x"]).to(DEV)
    ln = synth.layernorm_inputs(64, 12289, seed=k, mean=3.0, std=2.0)
    lx, lg, lb = (torch.from_numpy(ln[n]).to(DEV) for n in ("x", "gamma", "beta"))
    ce = synth.cross_entropy_inputs(256, 3072, seed=k)
    cx, cl = torch.from_numpy(ce["logits"]).to(DEV), torch.from_numpy(ce["labels"]).to(DEV)
    rm = synth.rmsnorm_inputs(768, 6144, seed=k)
    rx, rg = torch.from_numpy(rm["x"]).to(DEV), torch.from_numpy(rm["gamma"]).to(DEV)
    ws = torch.empty(lr.lr_workspace_query("layernorm", 64, 12289), dtype=torch.uint8, device=DEV)
    outs = dict(s=torch.empty_like(s), ln=torch.empty_like(lx), ce=torch.empty(256, device=DEV),
                rm=torch.empty_like(rx))

    def run(stream):
        sh = stream.cuda_stream
        lr.check(lr.lr_softmax_f32(s, outs["s"], 37, 1537, 0, sh), "softmax")
        lr.check(lr.lr_layernorm_f32(lx, lg, lb, outs["ln"], 64, 12289, 1e-5, 0, sh, workspace=ws), "layernorm")
        lr.check(lr.lr_cross_entropy_f32(cx, cl, outs["ce"], 256, 3072, 0, sh), "cross_entropy")
        lr.check(lr.lr_rmsnorm_f32(rx, rg, outs["rm"], 768, 6144, 1e-6, 0, sh), "rmsnorm")

    return run, outs


def test_concurrent_calls_from_host_threads():
    cases = [make_case(k) for k in range(THREADS)]
    # each case alone, on the current stream: the expected bits
    expected = []
    for run, outs in cases:
        run(torch.cuda.current_stream())
        torch.cuda.synchronize()
        expected.append({n: t.clone() for n, t in outs.items()})
        for t in outs.values():
            t.fill_(float("nan"))
    torch.cuda.synchronize()
    errors = []
    barrier = threading.Barrier(THREADS)

    def worker(k):
        try:
            run, _ = cases[k]
            stream = torch.cuda.Stream(device=DEV)
            barrier.wait()
            for _ in range(ITERS):
                run(stream)
            stream.synchronize()
        except Exception as e:  # reported below; a thread's exception does not fail the test by itself
            errors.append((k, repr(e)))

    print(f"\n[gpu] {THREADS} host threads x {ITERS} iterations", flush=True)
    threads = [threading.Thread(target=worker, args=(k,)) for k in range(THREADS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for k, (_, outs) in enumerate(cases):
        for n, t in outs.items():
            assert torch.equal(t.view(torch.int32), expected[k][n].view(torch.int32)), (k, n)
