"""The C-ABI launches under HIP graph capture (torch.cuda.graph): the kernels
allocate nothing and issue no memset, so a captured sequence of launches
replays to the same bits as the eager calls.  Each replay is checked against
the eager result, with eager work and synchronisation between replays."""
import numpy as np
import pytest
import torch

import row_reductions_amd as lr
import synth
from gpu_util import DEV

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    inp = synth.layernorm_inputs(64, 12289, seed=2, mean=3.0, std=2.0)
    x = torch.from_numpy(inp["x"]).to(DEV)
    g, b = torch.from_numpy(inp["gamma"]).to(DEV), torch.from_numpy(inp["beta"]).to(DEV)
    s_in = torch.from_numpy(synth.softmax_inputs(37, 1537, seed=1, std=4.0)["x"]).to(DEV)
    r_in = torch.from_numpy(synth.rmsnorm_inputs(256, 3072, seed=3)["x"]).to(DEV)
    rg = torch.from_numpy(synth.rmsnorm_inputs(256, 3072, seed=3)["gamma"]).to(DEV)

    def launch_all(outs):
        sh = torch.cuda.current_stream().cuda_stream  # the capture stream while capturing
        lr.check(lr.lr_layernorm_f32(x, g, b, outs[0], 64, 12289, 1e-5, "unordered_tree", sh))
        lr.check(lr.lr_softmax_f32(s_in, outs[1], 37, 1537, "unordered_tree", sh))
        lr.check(lr.lr_rmsnorm_f32(r_in, rg, outs[2], 256, 3072, 1e-6, "ordered_fold", sh))
        lr.check(lr.lr_rmsnorm_f32(r_in, rg, outs[3], 256, 3072, 1e-6, "ordered_tree", sh))

    shapes = [(64, 12289), (37, 1537), (256, 3072), (256, 3072)]
    eager = [torch.empty(s, device=DEV) for s in shapes]
    launch_all(eager)
    torch.cuda.synchronize()
    outs = [torch.full(s, float("nan"), device=DEV) for s in shapes]
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            launch_all(outs)
    torch.cuda.synchronize()
    for rep in range(5):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int32), e.view(torch.int32)), rep
        launch_all(eager)  # eager work between replays
        torch.cuda.synchronize()
