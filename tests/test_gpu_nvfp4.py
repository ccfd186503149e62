"""Parity of the NVFP4 path (E2M1 elements, an E4M3 scale per 16, an fp32
scale per tensor) with the fp64 oracle, through the C ABI.  The elements
times their block scales are exact in fp16 and the fp16 products exact in
fp32, so the error is the fp32 sum's (1e-4 sum|a b|), the fp32 rounding of
gA gB and of the final multiply (2^-22 |x|), and one ulp of a bf16 / fp16
output (oracle.check_epi with alpha 1 and the tensor scales inside the
oracle's sums).  Unit block and tensor scales make everything exact: those
fp32 outputs must match bit for bit."""
import contextlib
import os

import numpy as np
import pytest
import torch

import tensor_core_matrix_amd as tcm
from oracle import oracle as orc
from tensor_core_matrix_amd import inputs as inp

pytestmark = pytest.mark.gpu

DEV = "cuda"
OUT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
GUARD = 256


@contextlib.contextmanager
def env(**kv):
    old = {k: os.environ.get(k) for k in kv}
    os.environ.update({k: str(v) for k, v in kv.items()})
    try:
        yield
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def make(M, N, K, seed):
    g = inp.generator(seed)
    return (inp.e2m1_codes(M, K, g), inp.e2m1_codes(N, K, g),
            inp.e4m3_scales((M, K // 16), g), inp.e4m3_scales((N, K // 16), g))


def run(a, b, sa, sb, ga, gb, odt):
    n = a.shape[0] * b.shape[0]
    buf = torch.full((n + 2 * GUARD,), float("nan"), dtype=OUT[odt], device=DEV)
    out = buf[GUARD:GUARD + n].view(a.shape[0], b.shape[0])
    tcm.gemm_nvfp4(a.to(DEV), b.to(DEV), sa.to(DEV), sb.to(DEV), ga, gb, out)
    torch.cuda.synchronize()
    canary = torch.cat([buf[:GUARD], buf[-GUARD:]]).float()
    assert bool(torch.isnan(canary).all()), "write outside the output"
    return out.cpu()


def check(gpu, ref, s, odt, what):
    ok, worst, nbad = orc.check_epi(gpu.double().numpy(), ref, 1.0, s, np.zeros_like(ref), odt)
    assert ok, f"{what}: {nbad} violations, worst err/bound {worst:.3g}"


@pytest.mark.parametrize("K", [640, 608, 1024])
@pytest.mark.parametrize("odt", ["f32", "bf16", "f16"])
def test_nvfp4_ragged(K, odt):
    M, N = 700, 520
    a, b, sa, sb = make(M, N, K, 1200 + K)
    # tensor scales that keep the results inside the fp16 range (65504)
    ga, gb = (0.3, -1.7) if odt != "f16" else (0.03, -0.17)
    ref, s = orc.gemm_nvfp4(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb), ga, gb)
    check(run(a, b, sa, sb, ga, gb, odt), ref, s, odt, f"nvfp4 K {K} {odt}")


# 22 / 23: 256 and 128 tiles with two scale bytes per half row and slice;
# 24 / 25: the same tiles with a row's scales of four slices in one load
# (K a multiple of 256: here three such groups per tile); 34: the 16 x 16
# kernel on 256-deep E2M1 slices (three slices per tile)
@pytest.mark.parametrize("variant,K", [(22, 352), (23, 352), (22, 768), (23, 768), (24, 768),
                                       (25, 768), (34, 768)])
def test_nvfp4_each_tile_with_persistent_grid(variant, K):
    M, N = 777, 645
    a, b, sa, sb = make(M, N, K, 1210 + variant)
    ref, s = orc.gemm_nvfp4(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb), 2.0, 0.75)
    with env(TCM_FORCE_VARIANT=variant, TCM_MAX_GRID=3):
        got = run(a, b, sa, sb, 2.0, 0.75, "bf16")
    check(got, ref, s, "bf16", f"variant {variant} K {K}")


@pytest.mark.parametrize("variant", [24, 25, 34])
def test_nvfp4_wide_form_declined(variant):
    """A wide variant asked for where K is not a multiple of 256, or where a
    scale tensor is only 2-byte aligned, runs the two-bytes-per-half form."""
    M, N = 300, 260
    for K, shift in [(352, 0), (512, 2)]:
        a, b, sa, sb = make(M, N, K, 1240 + K)
        ref, s = orc.gemm_nvfp4(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb), 1.5, 0.5)
        # scale_B at a 2-byte offset inside a larger buffer
        holder = torch.zeros(N * K // 16 + 16, dtype=torch.uint8, device=DEV)
        sb_dev = holder[shift:shift + N * K // 16].view(N, K // 16)
        sb_dev.copy_(sb.to(DEV))
        n = M * N
        buf = torch.full((n + 2 * GUARD,), float("nan"), dtype=torch.float32, device=DEV)
        out = buf[GUARD:GUARD + n].view(M, N)
        with env(TCM_FORCE_VARIANT=variant):
            tcm.gemm_nvfp4(a.to(DEV), b.to(DEV), sa.to(DEV), sb_dev, 1.5, 0.5, out)
        torch.cuda.synchronize()
        assert bool(torch.isnan(torch.cat([buf[:GUARD], buf[-GUARD:]])).all())
        check(out.cpu(), ref, s, "f32", f"variant {variant} K {K} scale offset {shift}")


@pytest.mark.parametrize("shape,variant", [((1, 1, 32), None), ((33, 17, 64), None),
                                           ((256, 256, 128), None), ((300, 260, 1024), None),
                                           ((300, 260, 1024), 34), ((256, 256, 256), 34)])
def test_nvfp4_unit_scales_exact(shape, variant):
    M, N, K = shape
    a, b, _, _ = make(M, N, K, 1220 + K)
    one = 0x38  # E4M3 1.0
    sa = torch.full((M, K // 16), one, dtype=torch.uint8)
    sb = torch.full((N, K // 16), one, dtype=torch.uint8)
    ref, _ = orc.gemm_nvfp4(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb), 1.0, 1.0)
    with env(**({"TCM_FORCE_VARIANT": variant} if variant else {})):
        got = run(a, b, sa, sb, 1.0, 1.0, "f32").double().numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("variant", [None, 34])
def test_nvfp4_block_scale_reaches_only_its_16(variant):
    """Changing one 16-element scale of A changes exactly row 5's outputs, and
    those as the oracle says (positions in K pinned by the oracle).  Variant
    34 spreads a lane's 32 K values over four K steps: every block of 16 of
    a 512-deep row is changed in turn there."""
    M, N, K = 64, 48, 256 if variant is None else 512
    a, b, _, _ = make(M, N, K, 1230)
    sa = torch.full((M, K // 16), 0x38, dtype=torch.uint8)
    sb = torch.full((N, K // 16), 0x38, dtype=torch.uint8)
    kv = {"TCM_FORCE_VARIANT": variant} if variant else {}
    with env(**kv):
        base = run(a, b, sa, sb, 1.0, 1.0, "f32").double().numpy()
    for q in ([7] if variant is None else range(K // 16)):
        sa2 = sa.clone()
        sa2[5, q] = 0x4C  # E4M3 3.5
        with env(**kv):
            got = run(a, b, sa2, sb, 1.0, 1.0, "f32").double().numpy()
        ref, _ = orc.gemm_nvfp4(inp.raw(a), inp.raw(b), inp.raw(sa2), inp.raw(sb), 1.0, 1.0)
        assert np.array_equal(got, ref), f"block {q}"
        assert np.array_equal(np.delete(got, 5, 0), np.delete(base, 5, 0)), f"block {q}"


@pytest.mark.parametrize("variant", [22, 24, 34])
@pytest.mark.parametrize("odt", ["bf16", "f16"])
def test_nvfp4_staged_epilogue(variant, odt):
    """The 256 x 256 NVFP4 kernels with N a multiple of 8: interior tiles stage
    their 16-bit output through LDS with alpha = gA gB applied as it is
    staged; the ragged last tile row takes the alpha/beta epilogue.  Every
    output against the oracle, with and without a persistent grid."""
    M, N, K = 777, 648, 768
    a, b, sa, sb = make(M, N, K, 1250 + variant)
    ga, gb = (2.0, 0.75) if odt == "bf16" else (0.03, -0.17)
    ref, s = orc.gemm_nvfp4(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb), ga, gb)
    for grid in (None, 3):
        kv = {"TCM_FORCE_VARIANT": variant}
        if grid:
            kv["TCM_MAX_GRID"] = grid
        with env(**kv):
            got = run(a, b, sa, sb, ga, gb, odt)
        check(got, ref, s, odt, f"variant {variant} {odt} grid {grid}")


@pytest.mark.parametrize("K", [256, 1024])
@pytest.mark.parametrize("odt", ["f32", "bf16"])
def test_nvfp4_16x16_tile_sequences(K, odt):
    """Variant 34 with one slice per tile (K 256) and with four, several tiles
    per workgroup (a grid of 5 for 12 tiles), every output against the
    oracle, and block-scale pieces of B row r offset from A's."""
    M, N = 768, 1024
    a, b, sa, sb = make(M, N, K, 1260 + K)
    ref, s = orc.gemm_nvfp4(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb), -0.5, 1.25)
    with env(TCM_FORCE_VARIANT=34, TCM_MAX_GRID=5):
        got = run(a, b, sa, sb, -0.5, 1.25, odt)
    check(got, ref, s, odt, f"variant 34 K {K} {odt}")
