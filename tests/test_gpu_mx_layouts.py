"""Parity of MXFP8 with operands in either arrangement and leading dimensions
(tcm_gemm_mx: A the M x K and B the K x N matrix of E4M3 elements, each row-
or column-major, E8M0 scales per 32 K values of a row of A and a column of
B) with the fp64 oracle (oracle_gemm_mx_ld) through the C ABI.

Operands sit in rows padded with the E4M3 NaN byte, so a read of a pad that
reaches a stored output poisons it; Out's pads and the guard zones around it
must stay NaN.  Acceptance is the MX rule (1e-4 sum|a b| for the fp32 sums,
plus one ulp of a bf16 output); all-ones elements give an exact closed form."""
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
OUT = {"f32": torch.float32, "bf16": torch.bfloat16}
R, C = orc.ROW_MAJOR, orc.COL_MAJOR
GUARD = 256
NAN8 = 0x7F  # E4M3 NaN


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


def stored(x, order, extra=0):
    """Storage (2-D uint8, NaN pads) of logical matrix x in `order`, leading
    dimension = the contiguous extent rounded up to 16 plus `extra` (a
    multiple of 16); returns (storage, leading dimension)."""
    inner = x.shape[1] if order == R else x.shape[0]
    ld = (inner + 15) // 16 * 16 + extra
    src = x if order == R else x.T
    st = torch.full((src.shape[0], ld), NAN8, dtype=torch.uint8)
    st[:, :inner] = src
    return st, ld


def view(st, order, rows, cols):
    """The logical rows x cols matrix as a strided view of its storage."""
    return st[:, :cols] if order == R else st[:, :rows].T


def make(M, N, K, seed):
    g = inp.generator(seed)
    a = inp.e4m3_normal((M, K), g).view(torch.uint8)       # logical A
    bt = inp.e4m3_normal((N, K), g).view(torch.uint8)      # logical B^T: row j = column j
    sa = inp.e8m0_scales((M, K // 32), g)
    sb = inp.e8m0_scales((N, K // 32), g)
    return a, bt, sa, sb


def run(a, bt, sa, sb, ao, bo, odt, extra=0, ldo_extra=0, scales=None):
    """tcm.gemm_mx on device copies; returns (Out, oracle ref, oracle abssum)."""
    M, K = a.shape
    N = bt.shape[0]
    ast, lda = stored(a, ao, extra)
    bst, ldb = stored(bt.T.contiguous(), bo, extra)     # B is K x N
    ref, s = orc.gemm_mx_ld(ast.numpy(), ao, lda, bst.numpy(), bo, ldb, inp.raw(sa),
                            inp.raw(sb), M, N, K)
    ad, bd = ast.to(DEV), bst.to(DEV)
    A = view(ad, ao, M, K)
    B = view(bd, bo, K, N)
    ldo = N + ldo_extra
    buf = torch.full((M * ldo + 2 * GUARD,), float("nan"), dtype=OUT[odt], device=DEV)
    out = buf[GUARD:GUARD + M * ldo].view(M, ldo)[:, :N]
    sad, sbd = scales if scales is not None else (sa.to(DEV), sb.to(DEV))
    tcm.gemm_mx(A, B, sad, sbd, out)
    torch.cuda.synchronize()
    full = buf[GUARD:GUARD + M * ldo].view(M, ldo)
    pads_ok = bool(torch.isnan(full[:, N:].float()).all())
    guards_ok = bool(torch.isnan(torch.cat([buf[:GUARD], buf[-GUARD:]]).float()).all())
    assert pads_ok and guards_ok, "write outside the output"
    return out.cpu(), ref, s


def check(gpu, ref, s, odt, what):
    ok, worst, nbad = orc.check(gpu.double().numpy(), ref, s, odt == "bf16")
    assert ok, f"{what}: {nbad} violations, worst err/bound {worst:.3g}"


# K = 544 leaves a 32-deep tail of the last 128-deep slice and makes the scale
# rows no whole number of words (byte-wise scale reads)
@pytest.mark.parametrize("ao", [R, C])
@pytest.mark.parametrize("bo", [R, C])
@pytest.mark.parametrize("shape", [(300, 260, 512), (128, 128, 128), (17, 9, 64), (1000, 700, 544)])
def test_mx_arrangements(ao, bo, shape):
    M, N, K = shape
    a, bt, sa, sb = make(M, N, K, 1300 + M + N + K + 2 * ao + bo)
    odt = "bf16" if (M + ao) % 2 else "f32"
    got, ref, s = run(a, bt, sa, sb, ao, bo, odt)
    check(got, ref, s, odt, f"A {'RC'[ao]} B {'RC'[bo]} {shape} {odt}")


# variants 26 (256 x 128 tiles) and 11 (128 x 128), forced
@pytest.mark.parametrize("variant", [26, 11])
@pytest.mark.parametrize("ao,bo", [(C, R), (R, R), (C, C), (R, C)])
def test_mx_arrangement_leading_dimensions_and_persistent_grid(ao, bo, variant):
    """Leading dimensions past the rows on every matrix (operand pads are NaN),
    and a grid of 3 workgroups walking many tiles each, for each tile."""
    M, N, K = 777, 645, 768
    a, bt, sa, sb = make(M, N, K, 1320 + 2 * ao + bo + variant)
    with env(TCM_MAX_GRID=3, TCM_FORCE_VARIANT=variant):
        got, ref, s = run(a, bt, sa, sb, ao, bo, "f32", extra=48, ldo_extra=24)
    check(got, ref, s, "f32", f"ld, A {'RC'[ao]} B {'RC'[bo]}, variant {variant}")


# the ping-pong kernel (variant 14) with an M/N-major operand, forced: K =
# 1024 (scales by 16-byte chunks), 640 (by words), 544 (byte by byte, and a
# 32-deep tail in the last 64-deep unit), on a persistent grid
@pytest.mark.parametrize("K", [1024, 640, 544])
@pytest.mark.parametrize("ao,bo", [(C, R), (C, C), (R, R)])
def test_mx_arrangement_pingpong(ao, bo, K):
    M, N = 600, 520
    a, bt, sa, sb = make(M, N, K, 1370 + K + 2 * ao + bo)
    odt = "bf16" if K == 640 else "f32"
    with env(TCM_MAX_GRID=3, TCM_FORCE_VARIANT=14):
        got, ref, s = run(a, bt, sa, sb, ao, bo, odt)
    check(got, ref, s, odt, f"ping-pong, A {'RC'[ao]} B {'RC'[bo]}, K {K}")


def test_mx_arrangement_unaligned_scales():
    """Scale tensors at odd addresses: the byte-wise scale reads."""
    M, N, K = 256, 384, 512
    a, bt, sa, sb = make(M, N, K, 1330)
    bufa = torch.zeros(sa.numel() + 1, dtype=torch.uint8, device=DEV)
    bufb = torch.zeros(sb.numel() + 3, dtype=torch.uint8, device=DEV)
    va, vb = bufa[1:].view(M, K // 32), bufb[3:].view(N, K // 32)
    va.copy_(sa)
    vb.copy_(sb)
    got, ref, s = run(a, bt, sa, sb, C, R, "bf16", scales=(va, vb))
    check(got, ref, s, "bf16", "unaligned scales")


def test_mx_arrangement_all_ones_closed_form():
    """E4M3 1.0 everywhere, random scales: Out[i][j] = sum_q 32 * 2^(sA[i][q] +
    sB[j][q]) exactly, whatever the arrangement."""
    M, N, K = 200, 136, 384
    g = inp.generator(1340)
    a = torch.full((M, K), 0x38, dtype=torch.uint8)
    bt = torch.full((N, K), 0x38, dtype=torch.uint8)
    sa, sb = inp.e8m0_scales((M, K // 32), g), inp.e8m0_scales((N, K // 32), g)
    want = (32 * torch.exp2((sa.double() - 127)[:, None, :] + (sb.double() - 127)[None, :, :])).sum(-1)
    for ao, bo in [(C, R), (C, C), (R, R)]:
        got, _, _ = run(a, bt, sa, sb, ao, bo, "f32")
        assert torch.equal(got.double(), want), f"A {'RC'[ao]} B {'RC'[bo]}"


def test_mx_arrangement_large_full_output():
    """4096^3 with A column-major and B row-major (both operands M/N-major),
    every output against the oracle."""
    M = N = K = 4096
    a, bt, sa, sb = make(M, N, K, 1350)
    ast, lda = stored(a, C)
    bst, ldb = stored(bt.T.contiguous(), R)
    A = view(ast.to(DEV), C, M, K)
    B = view(bst.to(DEV), R, K, N)
    out = tcm.gemm_mx(A, B, sa.to(DEV), sb.to(DEV), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, s = orc.gemm_mx_ld(ast.numpy(), C, lda, bst.numpy(), R, ldb, inp.raw(sa), inp.raw(sb),
                            M, N, K)
    check(out.cpu(), ref, s, "bf16", "4096 full")


def test_mx_dense_tn_through_the_general_entry_is_the_tn_product():
    """Dense TN storage through tcm_gemm_mx runs tcm_gemm_mx_fp8's kernels:
    the outputs agree bit for bit."""
    M, N, K = 640, 384, 1024
    a, bt, sa, sb = make(M, N, K, 1360)
    ad, btd, sad, sbd = a.to(DEV), bt.to(DEV), sa.to(DEV), sb.to(DEV)
    want = tcm.gemm_mx_fp8(ad, btd, sad, sbd, out_dtype=torch.float32)
    got = tcm.gemm_mx(ad, btd.t(), sad, sbd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(got, want)


def test_k_zero_writes_zeros_every_block_scaled_entry():
    """K = 0: every output is the empty sum, 0, for each block-scaled entry
    (no operand or scale byte is read)."""
    M, N = 300, 260
    u8 = dict(dtype=torch.uint8, device=DEV)

    def fresh(dt=torch.float32):
        return torch.full((M, N), float("nan"), dtype=dt, device=DEV)

    outs = []
    o = fresh()
    tcm.gemm_mx_fp8(torch.empty(M, 0, **u8), torch.empty(N, 0, **u8), torch.empty(M, 0, **u8),
                    torch.empty(N, 0, **u8), o)
    outs.append(("mx_fp8", o))
    o = fresh()
    tcm.gemm_mx_fp4(torch.empty(M, 0, **u8), torch.empty(N, 0, **u8), torch.empty(M, 0, **u8),
                    torch.empty(N, 0, **u8), o)
    outs.append(("mx_fp4", o))
    o = fresh()
    tcm.gemm_mx_fp6(torch.empty(M, 0, **u8), torch.empty(N, 0, **u8), torch.empty(M, 0, **u8),
                    torch.empty(N, 0, **u8), o)
    outs.append(("mx_fp6", o))
    o = fresh(torch.float16)
    tcm.gemm_nvfp4(torch.empty(M, 0, **u8), torch.empty(N, 0, **u8), torch.empty(M, 0, **u8),
                   torch.empty(N, 0, **u8), 2.0, 3.0, o)
    outs.append(("nvfp4", o))
    o = fresh()
    # general MX entry: A column-major, B row-major, leading dimensions 16
    A = torch.empty(0, 16 * ((M + 15) // 16), **u8)[:, :M].t()
    B = torch.empty(0, 16 * ((N + 15) // 16), **u8)[:, :N]
    tcm.gemm_mx(A, B, torch.empty(M, 0, **u8), torch.empty(N, 0, **u8), o)
    outs.append(("mx general", o))
    torch.cuda.synchronize()
    for name, o in outs:
        assert bool((o == 0).all()), name
