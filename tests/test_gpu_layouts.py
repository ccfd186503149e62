"""Parity of the general form Out = alpha * (A . B) + beta * C with operands in
either arrangement (row- or column-major A and B) and leading dimensions on
every matrix, against the fp64 oracle through the C ABI (tcm_gemm).

Operands sit in NaN-padded rows (leading dimension past the row), so a read
of a pad poisons the result; Out's pads and the guard zones around it must
stay NaN.  Acceptance is the epilogue rule (|alpha| 1e-4 sum|a b| for the
fp32 sums, 2^-22 for the fp32 combine, one ulp of a bf16 / fp16 output);
quarter-integer operands with power-of-two alpha / beta are exact, so fp32
outputs must match bit for bit."""
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
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
ORC = {torch.float32: orc.F32, torch.bfloat16: orc.BF16, torch.float16: orc.F16}
R, C = orc.ROW_MAJOR, orc.COL_MAJOR
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


def stored(x, order, extra):
    """Storage (2-D, NaN pads) of logical matrix x in `order` with a leading
    dimension of the contiguous extent rounded up to 8, plus `extra` (a
    multiple of 8); returns (storage, leading dimension)."""
    inner = x.shape[1] if order == R else x.shape[0]
    ld = (inner + 7) // 8 * 8 + extra
    src = x if order == R else x.T
    st = torch.full((src.shape[0], ld), float("nan"), dtype=x.dtype)
    st[:, :inner] = src
    return st, ld


def view(st, order, rows, cols):
    """The logical rows x cols matrix as a strided view of its storage."""
    return st[:, :cols] if order == R else st[:, :rows].T


def run(a, ao, b, bo, c, alpha, beta, odt, extra=8, oextra=3):
    """Out from the GPU, and what the oracle expects.  a: M x K, b: K x N
    logical matrices (CPU tensors)."""
    M, K = a.shape
    N = b.shape[1]
    ast, lda = stored(a, ao, extra)
    bst, ldb = stored(b, bo, extra)
    ldo = N + oextra
    nbuf = M * ldo
    buf = torch.full((nbuf + 2 * GUARD,), float("nan"), dtype=TD[odt], device=DEV)
    out = buf[GUARD:GUARD + nbuf].view(M, ldo)[:, :N]
    ad, bd = ast.to(DEV), bst.to(DEV)
    cd = None
    if c is not None:
        cpad = torch.full((M, N + 5), float("nan"), dtype=c.dtype)
        cpad[:, :N] = c
        cd = cpad.to(DEV)[:, :N]
    tcm.gemm(view(ad, ao, M, K), view(bd, bo, K, N), cd, out, alpha, beta)
    torch.cuda.synchronize()
    host = buf.cpu()
    assert torch.isnan(torch.cat([host[:GUARD], host[-GUARD:]]).float()).all(), "write outside Out"
    if oextra:
        pads = host[GUARD:GUARD + nbuf].view(M, ldo)[:, N:]
        assert torch.isnan(pads.float()).all(), "write into Out's row padding"
    ref, s = orc.gemm_ld(ORC[a.dtype], inp.raw(ast), ao, lda, inp.raw(bst), bo, ldb, M, N, K)
    if c is None:
        ex, bc = orc.axpby(alpha, ref), np.zeros_like(ref)
    else:
        ex, bc = orc.axpby(alpha, ref, beta, inp.raw(c), ORC[c.dtype]), beta * c.double().numpy()
    return out.cpu(), ex, s, bc


def check(gpu, ex, alpha, s, bc, odt, what):
    ok, worst, nbad = orc.check_epi(gpu.double().numpy(), ex, alpha, s, bc, odt)
    assert ok, f"{what}: {nbad} violations, worst err/bound {worst:.3g}"


def operands(M, N, K, dt, seed, sigma=1.0):
    g = inp.generator(seed)
    return inp.normal((M, K), g, sigma, TD[dt]), inp.normal((K, N), g, sigma, TD[dt])


ORDERS = [(R, C), (R, R), (C, C), (C, R)]
IDS = {(R, C): "TN", (R, R): "Arow-Brow", (C, C): "Acol-Bcol", (C, R): "Acol-Brow"}


@pytest.mark.parametrize("orders", ORDERS, ids=lambda o: IDS[o])
@pytest.mark.parametrize("shape", [(1100, 600, 1000), (256, 256, 64), (300, 264, 72), (17, 9, 8),
                                   (1003, 999, 136)])
def test_orders_product(orders, shape):
    """alpha 1, beta 0, fp32 out: the plain kernel family for TN, the
    M/N-major kernels otherwise; ragged M and N, K tails."""
    M, N, K = shape
    a, b = operands(M, N, K, "bf16", 800 + M + N + K)
    got, ex, s, bc = run(a, orders[0], b, orders[1], None, 1.0, 0.0, "f32")
    check(got, ex, 1.0, s, bc, "f32", f"{IDS[orders]} {shape}")


@pytest.mark.parametrize("orders", ORDERS, ids=lambda o: IDS[o])
@pytest.mark.parametrize("odt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_orders_axpby(orders, odt, dt):
    M, N, K = 700, 520, 200
    a, b = operands(M, N, K, dt, 820)
    c = inp.normal((M, N), inp.generator(821), 3.0, torch.float32)
    got, ex, s, bc = run(a, orders[0], b, orders[1], c, -0.75, 1.5, odt)
    check(got, ex, -0.75, s, bc, odt, f"{IDS[orders]} {dt} -> {odt}")


@pytest.mark.parametrize("orders", ORDERS, ids=lambda o: IDS[o])
@pytest.mark.parametrize("variant", [19, 2])
def test_forced_tiles_and_persistent_grid(orders, variant):
    """Both M/N-major tiles (256 x 256 split-3, 128 x 128) with a capped grid,
    so workgroups carry several tiles and the copy stream crosses tiles."""
    M, N, K = 777, 645, 328
    a, b = operands(M, N, K, "f16", 830 + variant)
    with env(TCM_FORCE_VARIANT=variant, TCM_MAX_GRID=3):
        got, ex, s, bc = run(a, orders[0], b, orders[1], None, 1.0, 0.0, "bf16")
    check(got, ex, 1.0, s, bc, "bf16", f"{IDS[orders]} variant {variant}")


@pytest.mark.parametrize("K", [1, 5, 13, 67, 130])
def test_free_k_with_both_operands_mn_major(K):
    """Column-major A with row-major B: K need not be a multiple of 8 (rows
    past K read as zeros through the per-slice bound)."""
    M, N = 300, 200
    a, b = operands(M, N, K, "bf16", 840 + K)
    got, ex, s, bc = run(a, C, b, R, None, 1.0, 0.0, "f32")
    check(got, ex, 1.0, s, bc, "f32", f"K {K}")


def test_k_zero_is_beta_c():
    M, N = 130, 70
    a = torch.zeros(M, 0, dtype=torch.bfloat16)
    b = torch.zeros(0, N, dtype=torch.bfloat16)
    c = inp.normal((M, N), inp.generator(850), 1.0, torch.bfloat16)
    got, ex, s, bc = run(a, C, b, R, c, 2.0, 0.5, "f32")
    assert np.array_equal(got.double().numpy(), ex)


@pytest.mark.parametrize("orders", ORDERS, ids=lambda o: IDS[o])
def test_exact_quarter_integers(orders):
    M, N, K = 640, 384, 512
    g = inp.generator(860)
    a = inp.quarter_integers((M, K), g, torch.float16)
    b = inp.quarter_integers((K, N), g, torch.float16)
    c = inp.quarter_integers((M, N), g, torch.float32) * 64
    got, ex, _, _ = run(a, orders[0], b, orders[1], c, 2.0, -0.5, "f32")
    assert np.array_equal(got.double().numpy(), ex)


def test_in_place_with_leading_dimension():
    M, N, K = 333, 260, 96
    a, b = operands(M, N, K, "bf16", 870)
    ast, lda = stored(a, C, 16)
    bst, ldb = stored(b, R, 0)
    o = torch.full((M, N + 12), float("nan"), dtype=torch.float32)
    c = inp.normal((M, N), inp.generator(871), 2.0, torch.float32)
    o[:, :N] = c
    od = o.to(DEV)
    tcm.gemm(view(ast.to(DEV), C, M, K), view(bst.to(DEV), R, K, N), od[:, :N], od[:, :N],
             0.5, -2.0)
    torch.cuda.synchronize()
    host = od.cpu()
    assert torch.isnan(host[:, N:]).all()
    ref, s = orc.gemm_ld(orc.BF16, inp.raw(ast), C, lda, inp.raw(bst), R, ldb, M, N, K)
    ex = orc.axpby(0.5, ref, -2.0, inp.raw(c), orc.F32)
    check(host[:, :N], ex, 0.5, s, -2.0 * c.double().numpy(), "f32", "in place")


@pytest.mark.parametrize("orders", [(R, R), (C, C), (C, R)], ids=lambda o: IDS[o])
def test_large_full_output(orders):
    """4096^3 at the default 256 x 256 tile, every output against the oracle."""
    M = N = K = 4096
    a, b = operands(M, N, K, "bf16", 880, 0.1)
    ao, bo = orders
    ast, lda = stored(a, ao, 0)
    bst, ldb = stored(b, bo, 0)
    out = tcm.gemm(view(ast.to(DEV), ao, M, K), view(bst.to(DEV), bo, K, N),
                   out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, s = orc.gemm_ld(orc.BF16, inp.raw(ast), ao, lda, inp.raw(bst), bo, ldb, M, N, K)
    check(out.cpu(), orc.axpby(1.0, ref), 1.0, s, np.zeros_like(ref), "bf16",
          f"{IDS[orders]} 4096")


@pytest.mark.parametrize("ao,bo", [(R, C), (C, R)])
def test_k_zero_general_form_is_beta_c(ao, bo):
    """K = 0: the product is the empty sum, so Out = op(beta * C) exactly
    (power-of-two beta), for K-major and M/N-major operands alike."""
    M, N = 300, 260
    g = inp.generator(1400 + ao)
    c = inp.normal((M, N), g, 1.0, torch.float32)
    a_st = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV) if ao == C else \
        torch.empty(M, 8, dtype=torch.bfloat16, device=DEV)
    b_st = torch.empty(0, 264, dtype=torch.bfloat16, device=DEV) if bo == R else \
        torch.empty(N, 8, dtype=torch.bfloat16, device=DEV)
    a = a_st[:, :0] if ao == R else torch.empty(0, 304, dtype=torch.bfloat16, device=DEV)[:, :M].t()
    b = b_st[:, :N] if bo == R else b_st[:, :0].t()
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    tcm.gemm(a, b, c.to(DEV), out, alpha=3.0, beta=-0.5, op="relu")
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.relu(-0.5 * c))
