"""Entries captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

An entry makes no allocation, synchronization or memset inside a call (the
device properties are read once per device, before capture here), so it can
be recorded into a graph.  Each replay, with eager work between replays,
must give the eager result bit for bit, and a replay after the inputs were
overwritten in place must give the product of the new inputs.
"""
import pytest
import torch

import tensor_core_matrix_amd as tcm
from tensor_core_matrix_amd import inputs as inp

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_graph_replays_match_eager():
    g = inp.generator(950)
    M, N, K = 512, 384, 640
    a = inp.normal((M, K), g, 1.0, torch.bfloat16).to(DEV)
    b = inp.normal((N, K), g, 1.0, torch.bfloat16).to(DEV)
    a2 = inp.normal((M, K), g, 1.0, torch.bfloat16).to(DEV)
    xa = inp.e4m3_normal((M, K), g).to(DEV)
    xb = inp.e4m3_normal((N, K), g).to(DEV)
    sa = inp.e8m0_scales((M, K // 32), g).to(DEV)
    sb = inp.e8m0_scales((N, K // 32), g).to(DEV)
    c = inp.normal((M, N), g, 1.0, torch.bfloat16).to(DEV)

    o1 = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    o2 = torch.empty(M, N, dtype=torch.float32, device=DEV)
    o3 = torch.empty(M, N, dtype=torch.float32, device=DEV)

    def calls():
        tcm.gemm_tn(a, b, o1)
        tcm.gemm_mx_fp8(xa, xb, sa, sb, o2)
        tcm.gemm_tn_ex(a, b, c=c, out=o3, alpha=0.5, beta=-2.0)

    calls()  # eager, also reads the device properties before capture
    torch.cuda.synchronize()
    e1, e2, e3 = o1.clone(), o2.clone(), o3.clone()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):  # captures on its own stream, made current
        calls()
    torch.cuda.synchronize()

    for r in range(3):
        for o in (o1, o2, o3):
            o.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o1, e1), f"replay {r}: bf16 product"
        assert torch.equal(o2, e2), f"replay {r}: MXFP8 product"
        assert torch.equal(o3, e3), f"replay {r}: alpha/beta form"

    # the graph reads the inputs' memory at replay time
    a.copy_(a2)
    graph.replay()
    torch.cuda.synchronize()
    r1 = torch.empty_like(o1)
    tcm.gemm_tn(a2, b, r1)
    torch.cuda.synchronize()
    assert torch.equal(o1, r1)
