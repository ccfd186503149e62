"""Parity of the MXFP4 path (E2M1 elements, E8M0 scales per 32) with the fp64
oracle, through the C ABI.  Same acceptance rule as the other products:
|gpu - ref| <= 1e-4 * sum_k |a_ik b_jk| (+ one bf16 ulp for bf16 output).
Unit scales make every product and partial sum exact in fp32, so those cases
must match bit for bit.  The scale tensors are read three ways depending on
K and alignment (byte by byte, 32-bit words, 16-byte pieces): the shapes
below reach each of them."""
import numpy as np
import pytest
import torch

import tensor_core_matrix_amd as tcm
from oracle import oracle as orc
from tensor_core_matrix_amd import inputs as inp

pytestmark = pytest.mark.gpu

DEV = "cuda"
OUT = {"f32": torch.float32, "bf16": torch.bfloat16}
GUARD = 256


def run_fp4(a, b, sa, sb, out_dtype):
    n = a.shape[0] * b.shape[0]
    buf = torch.full((n + 2 * GUARD,), float("nan"), dtype=OUT[out_dtype], device=DEV)
    out = buf[GUARD:GUARD + n].view(a.shape[0], b.shape[0])
    tcm.gemm_mx_fp4(a.to(DEV), b.to(DEV), sa.to(DEV), sb.to(DEV), out)
    torch.cuda.synchronize()
    canary = torch.cat([buf[:GUARD], buf[-GUARD:]]).float()
    assert bool(torch.isnan(canary).all()), "write outside the output"
    return out.cpu()


def check(gpu, ref, s, out_dtype, what):
    ok, worst, nbad = orc.check(gpu.double().numpy(), ref, s, out_dtype == "bf16")
    assert ok, f"{what}: {nbad} violations, worst err/bound {worst:.3g}"


def make(M, N, K, seed, lo=-4, hi=4):
    g = inp.generator(seed)
    a = inp.e2m1_codes(M, K, g)
    b = inp.e2m1_codes(N, K, g)
    sa = inp.e8m0_scales((M, K // 32), g, lo, hi)
    sb = inp.e8m0_scales((N, K // 32), g, lo, hi)
    return a, b, sa, sb


@pytest.fixture
def grid_cap(monkeypatch):
    def _set(n):
        if n is None:
            monkeypatch.delenv("TCM_MAX_GRID", raising=False)
        else:
            monkeypatch.setenv("TCM_MAX_GRID", str(n))
    return _set


# K = 640: word-wise scales; 608: byte-wise (19 blocks, a 96-deep K tail);
# 1536: 16-byte scale pieces, three 512-deep chunks per tile
@pytest.mark.parametrize("K", [640, 608, 1536])
@pytest.mark.parametrize("odt", ["f32", "bf16"])
def test_mxfp4_ragged(K, odt, grid_cap):
    M, N = 700, 520
    a, b, sa, sb = make(M, N, K, 500 + K)
    ref, s = orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb), dtype=orc.E2M1)
    grid_cap(None)
    check(run_fp4(a, b, sa, sb, odt), ref, s, odt, f"mxfp4 K {K} {odt}")
    # three persistent workgroups, several tiles each
    grid_cap(3)
    check(run_fp4(a, b, sa, sb, odt), ref, s, odt, f"mxfp4 K {K} {odt} grid 3")


@pytest.mark.parametrize("shape", [(1, 1, 32), (33, 17, 64), (256, 256, 128), (300, 260, 1024)])
def test_mxfp4_unit_scales_exact(shape):
    M, N, K = shape
    a, b, _, _ = make(M, N, K, 600 + K)
    sa = torch.full((M, K // 32), 127, dtype=torch.uint8)
    sb = torch.full((N, K // 32), 127, dtype=torch.uint8)
    ref, _ = orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb), dtype=orc.E2M1)
    got = run_fp4(a, b, sa, sb, "f32").double().numpy()
    assert np.array_equal(got, ref)


def test_mxfp4_scale_reaches_only_its_block():
    """One scale per (row, block): raising one scale of A changes exactly the
    terms of that row and block (positions in K pinned by the oracle)."""
    M, N, K = 64, 48, 256
    a, b, _, _ = make(M, N, K, 610)
    sa = torch.full((M, K // 32), 127, dtype=torch.uint8)
    sb = torch.full((N, K // 32), 127, dtype=torch.uint8)
    base = run_fp4(a, b, sa, sb, "f32").double().numpy()
    sa2 = sa.clone()
    sa2[5, 3] = 127 + 4
    got = run_fp4(a, b, sa2, sb, "f32").double().numpy()
    ref, _ = orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw(sa2), inp.raw(sb), dtype=orc.E2M1)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.delete(got, 5, 0), np.delete(base, 5, 0))
