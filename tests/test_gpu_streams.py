"""Stream semantics and concurrent callers of the C ABI on the GPU.

Every entry launches on the caller's stream (the binding passes torch's
current stream) and does not synchronize, so work queued before it on the
same stream is seen and work queued after it sees its output.  The library
keeps no per-call state, so host threads calling it at once, each on its own
stream, get the results they would get alone.
"""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

import tensor_core_matrix_amd as tcm
from oracle import oracle as orc
from tensor_core_matrix_amd import inputs as inp

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _check(out, ref, s, bf16_out, what):
    ok, worst, nbad = orc.check(out.double().numpy(), ref, s, bf16_out)
    assert ok, f"{what}: {nbad} elements over the bound (worst {worst:.3g})"


def test_launch_is_ordered_on_the_callers_stream():
    """Inputs are produced on a side stream behind a ~1 ms device spin; the
    product and a copy of it are queued on the same stream without any
    synchronization in between.  Launching anywhere but that stream would
    read the zero-filled inputs."""
    M, N, K = 384, 320, 512
    g = inp.generator(901)
    a = inp.normal((M, K), g, 1.0, torch.bfloat16)
    b = inp.normal((N, K), g, 1.0, torch.bfloat16)
    ref, s = orc.gemm_tn(orc.BF16, inp.raw(a), inp.raw(b))
    src_a, src_b = a.to(DEV), b.to(DEV)
    ad = torch.zeros_like(src_a)
    bd = torch.zeros_like(src_b)
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        torch.cuda._sleep(2_000_000)
        ad.copy_(src_a)
        bd.copy_(src_b)
        tcm.gemm_tn(ad, bd, out)
        seen = out.clone()
    side.synchronize()
    _check(seen.cpu(), ref, s, False, "side stream")


def _job(kind, seed):
    g = inp.generator(seed)
    if kind == "bf16":
        M, N, K = 520, 260, 384
        a = inp.normal((M, K), g, 1.0, torch.bfloat16)
        b = inp.normal((N, K), g, 1.0, torch.bfloat16)
        ref, s = orc.gemm_tn(orc.BF16, inp.raw(a), inp.raw(b))

        def run():
            out = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
            tcm.gemm_tn(a.to(DEV), b.to(DEV), out)
            return out
        return run, ref, s, True
    if kind == "f16":
        M, N, K = 300, 700, 256
        a = inp.normal((M, K), g, 1.0, torch.float16)
        b = inp.normal((N, K), g, 1.0, torch.float16)
        ref, s = orc.gemm_tn(orc.F16, inp.raw(a), inp.raw(b))

        def run():
            out = torch.empty(M, N, dtype=torch.float32, device=DEV)
            tcm.gemm_tn(a.to(DEV), b.to(DEV), out)
            return out
        return run, ref, s, False
    # MXFP8
    M, N, K = 256, 384, 640
    a = inp.e4m3_normal((M, K), g)
    b = inp.e4m3_normal((N, K), g)
    sa = inp.e8m0_scales((M, K // 32), g)
    sb = inp.e8m0_scales((N, K // 32), g)
    ref, s = orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb))

    def run():
        out = torch.empty(M, N, dtype=torch.float32, device=DEV)
        tcm.gemm_mx_fp8(a.to(DEV), b.to(DEV), sa.to(DEV), sb.to(DEV), out)
        return out
    return run, ref, s, False


def test_concurrent_callers_on_their_own_streams():
    """Four host threads, each with its own stream, call three entries
    (bf16, f16 -> f32, MXFP8) three times each at once; every result matches
    the oracle."""
    kinds = ["bf16", "f16", "mx", "bf16"]
    jobs = [_job(k, 910 + i) for i, k in enumerate(kinds)]
    torch.cuda.synchronize()

    def worker(i):
        run = jobs[i][0]
        st = torch.cuda.Stream()
        outs = []
        with torch.cuda.stream(st):
            for _ in range(3):
                outs.append(run())
        st.synchronize()
        return [o.float().cpu() for o in outs]

    with cf.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        results = list(ex.map(worker, range(len(jobs))))
    for (run, ref, s, bf16_out), outs, kind in zip(jobs, results, kinds):
        for r, out in enumerate(outs):
            _check(out, ref, s, bf16_out, f"{kind} call {r}")
        # a repeated call gives the same bits
        assert all(np.array_equal(outs[0].numpy(), o.numpy()) for o in outs[1:])
