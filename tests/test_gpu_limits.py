"""The documented size limits, at the limit, on the GPU: K = 2^20 (the largest
K any entry takes) and a leading dimension of 2^21 (the largest for A and
B).  All-ones operands with unit scales make the product an exact closed
form (every partial sum is an integer below 2^24), so the fp32 outputs must
equal K bit for bit; no oracle is needed."""
import pytest
import torch

import tensor_core_matrix_amd as tcm

pytestmark = pytest.mark.gpu

DEV = "cuda"
KMAX = 1 << 20


def test_bf16_largest_k():
    a = torch.ones(256, KMAX, dtype=torch.bfloat16, device=DEV)
    b = torch.ones(256, KMAX, dtype=torch.bfloat16, device=DEV)
    out = tcm.gemm_tn(a, b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert bool((out == KMAX).all())


def test_mxfp8_largest_k_tn_and_m_major():
    M = N = 256
    one = torch.full((M, KMAX), 0x38, dtype=torch.uint8, device=DEV)     # E4M3 1.0
    unit = torch.full((M, KMAX // 32), 127, dtype=torch.uint8, device=DEV)  # E8M0 1.0
    out = tcm.gemm_mx_fp8(one, one, unit, unit, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert bool((out == KMAX).all())
    # A stored K x M (M-major, K * lda = 2^28), B stored K x N (N-major)
    a_km = torch.full((KMAX, M), 0x38, dtype=torch.uint8, device=DEV)
    out = tcm.gemm_mx(a_km.t(), a_km, unit, unit, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert bool((out == KMAX).all())


def test_nvfp4_largest_k():
    M = N = 256
    ones = torch.full((M, KMAX // 2), 0x22, dtype=torch.uint8, device=DEV)   # E2M1 1.0, 1.0
    unit = torch.full((M, KMAX // 16), 0x38, dtype=torch.uint8, device=DEV)  # E4M3 1.0
    out = torch.empty(M, N, dtype=torch.float32, device=DEV)
    tcm.gemm_nvfp4(ones, ones, unit, unit, 1.0, 1.0, out)
    torch.cuda.synchronize()
    assert bool((out == KMAX).all())


def test_largest_leading_dimension():
    """Row-major A with lda = 2^21 (rows 4 MiB apart): only the first K
    values of each row are A; the rest of the row is NaN and must not be
    read."""
    M, N, K, LD = 16, 24, 64, 1 << 21
    st = torch.full((M, LD), float("nan"), dtype=torch.bfloat16, device=DEV)
    st[:, :K] = 1.0
    a = st[:, :K]
    b = torch.ones(K, N, dtype=torch.bfloat16, device=DEV)
    out = tcm.gemm(a, b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert tcm.order_ld(a) == (tcm.ROW_MAJOR, LD)
    assert bool((out == K).all())
