"""Parity of the MXFP6 path (FP6 E2M3 or E3M2 codes packed four per three
bytes, E8M0 scales per 32) with the fp64 oracle, through the C ABI.  Same
acceptance rule as the other products: |gpu - ref| <= 1e-4 * sum_k |a_ik b_jk|
(+ one bf16 ulp for bf16 output).  With unit scales, E2M3 products and sums
up to K = 1024 are exact in fp32, so those cases must match bit for bit.  The
shapes reach all three ways of reading the scales (bytes: K = 576, 32-bit
words: K = 640, 16-byte pieces: K = 1536), each on the ping-pong kernels:
128-deep units (variant 27, the default where scales are read as words;
K = 576 leaves its last unit half empty) and 64-deep units (variant 21);
and, where scales come as 16-byte pieces (K = 1536, 1024), on the default
there, the 16 x 16 x 128 kernel (variant 36; forced on other shapes it gives
way to variant 27 or 21)."""
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


def run_fp6(a, b, sa, sb, out_dtype, elem):
    n = a.shape[0] * b.shape[0]
    buf = torch.full((n + 2 * GUARD,), float("nan"), dtype=OUT[out_dtype], device=DEV)
    out = buf[GUARD:GUARD + n].view(a.shape[0], b.shape[0])
    tcm.gemm_mx_fp6(a.to(DEV), b.to(DEV), sa.to(DEV), sb.to(DEV), out, elem=elem)
    torch.cuda.synchronize()
    canary = torch.cat([buf[:GUARD], buf[-GUARD:]]).float()
    assert bool(torch.isnan(canary).all()), "write outside the output"
    return out.cpu()


def check(gpu, ref, s, out_dtype, what):
    ok, worst, nbad = orc.check(gpu.double().numpy(), ref, s, out_dtype == "bf16")
    assert ok, f"{what}: {nbad} violations, worst err/bound {worst:.3g}"


def make(M, N, K, seed, lo=-4, hi=4):
    g = inp.generator(seed)
    a = inp.fp6_codes(M, K, g)
    b = inp.fp6_codes(N, K, g)
    sa = inp.e8m0_scales((M, K // 32), g, lo, hi)
    sb = inp.e8m0_scales((N, K // 32), g, lo, hi)
    return a, b, sa, sb


def oracle(a, b, sa, sb, elem):
    return orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb),
                       dtype=orc.DTYPE_NAMES[elem])


@pytest.fixture
def grid_cap(monkeypatch):
    def _set(n):
        if n is None:
            monkeypatch.delenv("TCM_MAX_GRID", raising=False)
        else:
            monkeypatch.setenv("TCM_MAX_GRID", str(n))
    return _set


@pytest.fixture(params=[27, 21, 36])
def variant(request, monkeypatch):
    monkeypatch.setenv("TCM_FORCE_VARIANT", str(request.param))
    return request.param


@pytest.mark.parametrize("K", [576, 640, 1536])
@pytest.mark.parametrize("odt", ["f32", "bf16"])
@pytest.mark.parametrize("elem", ["e2m3", "e3m2"])
def test_mxfp6_ragged(K, odt, elem, grid_cap, variant):
    M, N = 700, 520
    a, b, sa, sb = make(M, N, K, 1000 + K)
    ref, s = oracle(a, b, sa, sb, elem)
    grid_cap(None)
    check(run_fp6(a, b, sa, sb, odt, elem), ref, s, odt, f"mxfp6 {elem} K {K} {odt}")
    grid_cap(3)
    check(run_fp6(a, b, sa, sb, odt, elem), ref, s, odt, f"mxfp6 {elem} K {K} {odt} grid 3")


@pytest.mark.parametrize("shape", [(1, 1, 64), (33, 17, 64), (256, 256, 128), (300, 260, 1024)])
def test_mxfp6_unit_scales_exact(shape, variant):
    M, N, K = shape
    a, b, _, _ = make(M, N, K, 1100 + K)
    sa = torch.full((M, K // 32), 127, dtype=torch.uint8)
    sb = torch.full((N, K // 32), 127, dtype=torch.uint8)
    ref, _ = oracle(a, b, sa, sb, "e2m3")
    got = run_fp6(a, b, sa, sb, "f32", "e2m3").double().numpy()
    assert np.array_equal(got, ref)


def test_mxfp6_scale_reaches_only_its_block():
    M, N, K = 64, 48, 256
    a, b, _, _ = make(M, N, K, 1110)
    sa = torch.full((M, K // 32), 127, dtype=torch.uint8)
    sb = torch.full((N, K // 32), 127, dtype=torch.uint8)
    base = run_fp6(a, b, sa, sb, "f32", "e2m3").double().numpy()
    sa2 = sa.clone()
    sa2[5, 3] = 127 + 4
    got = run_fp6(a, b, sa2, sb, "f32", "e2m3").double().numpy()
    ref, _ = oracle(a, b, sa2, sb, "e2m3")
    assert np.array_equal(got, ref)
    assert np.array_equal(np.delete(got, 5, 0), np.delete(base, 5, 0))


@pytest.mark.parametrize("K", [512, 1024, 2560])
@pytest.mark.parametrize("elem", ["e2m3", "e3m2"])
def test_mxfp6_16x16_tile_sequences(K, elem, grid_cap, monkeypatch):
    """The 16 x 16 x 128 kernel forced on a ragged multi-tile shape: one, two
    and five scale chunks of 512 K per tile, every workgroup of a grid of 5
    walking several tiles (the last ragged in M and N), both outputs."""
    monkeypatch.setenv("TCM_FORCE_VARIANT", "36")
    M, N = 600, 1100
    a, b, sa, sb = make(M, N, K, 1200 + K)
    ref, s = oracle(a, b, sa, sb, elem)
    for cap in (None, 5):
        grid_cap(cap)
        for odt in ("f32", "bf16"):
            check(run_fp6(a, b, sa, sb, odt, elem), ref, s, odt, f"variant 36 {elem} K {K} {odt} grid {cap}")


def test_mxfp6_16x16_wide_block_scales(monkeypatch):
    """Variant 36 with every (row, block) scale of A and B drawn from
    2^-8 .. 2^8: a block whose scale reached another block's values, or
    values read from the wrong bytes of a 96-byte row slice, moves outputs
    by factors far outside the bound."""
    monkeypatch.setenv("TCM_FORCE_VARIANT", "36")
    M, N, K = 256, 256, 512
    a, b, sa, sb = make(M, N, K, 1300, -8, 8)
    for elem in ("e2m3", "e3m2"):
        ref, s = oracle(a, b, sa, sb, elem)
        check(run_fp6(a, b, sa, sb, "f32", elem), ref, s, "f32", f"variant 36 wide scales {elem}")
