"""Parity of the epilogue with a per-element operation, Out = op(alpha * (A . B)
+ beta * C), with the fp64 oracle through the C ABI (tcm_gemm).  Acceptance:
the fp32 sum and combine errors carried through op's largest slope, 2^-20
(|x| + |op(x)|) for op evaluated in fp32, and one ulp of a bf16 / fp16
output (oracle.check_op).  Values x = alpha * sum + beta * c span about
[-8, 8], where the operations bend."""
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
OPS = ["relu", "gelu_tanh", "gelu_erf", "silu"]
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


def case(M, N, K, seed, dt="bf16", c_dt="f32"):
    g = inp.generator(seed)
    a = inp.normal((M, K), g, 0.25, TD[dt])
    b = inp.normal((N, K), g, 0.25, TD[dt])     # B^T rows: b.T is the K x N matrix B
    c = inp.normal((M, N), g, 2.5, TD[c_dt])
    return a, b, c


def run(a, bt, c, alpha, beta, op, odt, b_row_major=False):
    """GPU Out for A = a (row-major) and B = bt^T, stored column-major (as bt)
    or row-major (a K x N copy); Out inside NaN guard zones."""
    M, N = a.shape[0], bt.shape[0]
    buf = torch.full((M * N + 2 * GUARD,), float("nan"), dtype=TD[odt], device=DEV)
    out = buf[GUARD:GUARD + M * N].view(M, N)
    bd = bt.T.contiguous().to(DEV) if b_row_major else bt.to(DEV).T
    tcm.gemm(a.to(DEV), bd, None if c is None else c.to(DEV), out, alpha, beta, op=op)
    torch.cuda.synchronize()
    host = buf.cpu()
    assert torch.isnan(torch.cat([host[:GUARD], host[-GUARD:]]).float()).all(), "write outside Out"
    return out.cpu()


def expect(a, bt, c, alpha, beta):
    ref, s = orc.gemm_tn(ORC[a.dtype], inp.raw(a), inp.raw(bt))
    if c is None:
        return orc.axpby(alpha, ref), s, np.zeros_like(ref)
    return orc.axpby(alpha, ref, beta, inp.raw(c), ORC[c.dtype]), s, beta * c.double().numpy()


def check(gpu, x, op, alpha, s, bc, odt, what):
    ok, worst, nbad = orc.check_op(gpu.double().numpy(), x, orc.OPS[op], alpha, s, bc, odt)
    assert ok, f"{what}: {nbad} violations, worst err/bound {worst:.3g}"


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("odt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("b_row_major", [False, True], ids=["TN", "B-row-major"])
def test_ops(op, odt, b_row_major):
    M, N, K = 700, 520, 200
    a, bt, c = case(M, N, K, 900 + orc.OPS[op])
    x, s, bc = expect(a, bt, c, 0.75, 1.25)
    got = run(a, bt, c, 0.75, 1.25, op, odt, b_row_major)
    check(got, x, op, 0.75, s, bc, odt, f"{op} -> {odt} {'NN' if b_row_major else 'TN'}")


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("variant", [19, 1, 2, 3])
def test_ops_each_tile_with_persistent_grid(op, variant):
    """Every tile the C-input kernels run (3, the 128 x 64 tile, is taken to
    128 x 128 for an operation), several tiles per workgroup; no C input."""
    M, N, K = 777, 645, 328
    a, bt, _ = case(M, N, K, 910 + variant, "f16")
    x, s, bc = expect(a, bt, None, -1.5, 0.0)
    with env(TCM_FORCE_VARIANT=variant, TCM_MAX_GRID=3):
        got = run(a, bt, None, -1.5, 0.0, op, "bf16")
    check(got, x, op, -1.5, s, bc, "bf16", f"{op} variant {variant}")


@pytest.mark.parametrize("shape", [(17, 9, 8), (1, 1, 8), (300, 264, 72), (256, 256, 64)])
def test_ops_small_and_ragged(shape):
    M, N, K = shape
    a, bt, c = case(M, N, K, 920 + M, "bf16", "bf16")
    x, s, bc = expect(a, bt, c, 1.0, -1.0)
    got = run(a, bt, c, 1.0, -1.0, "gelu_erf", "f32")
    check(got, x, "gelu_erf", 1.0, s, bc, "f32", f"{shape}")


def test_relu_exact_on_quarter_integers():
    """relu is exact and the sums of quarter-integer products are exact in
    fp32: the output is relu of the exact value, bit for bit."""
    M, N, K = 640, 384, 512
    g = inp.generator(930)
    a = inp.quarter_integers((M, K), g, torch.float16)
    bt = inp.quarter_integers((N, K), g, torch.float16)
    c = inp.quarter_integers((M, N), g, torch.float32) * 64
    x, _, _ = expect(a, bt, c, 2.0, -0.5)
    got = run(a, bt, c, 2.0, -0.5, "relu", "f32").double().numpy()
    assert np.array_equal(got, np.where(x > 0, x, 0.0))


def test_op_in_place():
    M, N, K = 520, 700, 128
    a, bt, c = case(M, N, K, 940)
    x, s, bc = expect(a, bt, c, 2.0, 0.5)
    cd = c.to(DEV)
    tcm.gemm(a.to(DEV), bt.to(DEV).T, cd, cd, 2.0, 0.5, op="silu")
    torch.cuda.synchronize()
    check(cd.cpu(), x, "silu", 2.0, s, bc, "f32", "in place")


def test_op_large_full_output():
    """4096^3 with alpha 8 and GELU (x Phi(x)), every output against the oracle."""
    M = N = K = 4096
    g = inp.generator(950)
    a = inp.normal((M, K), g, 0.05, torch.bfloat16)
    bt = inp.normal((N, K), g, 0.05, torch.bfloat16)
    out = tcm.gemm(a.to(DEV), bt.to(DEV).T, out_dtype=torch.bfloat16, alpha=8.0, op="gelu_erf")
    torch.cuda.synchronize()
    ref, s = orc.gemm_tn(orc.BF16, inp.raw(a), inp.raw(bt))
    check(out.cpu(), orc.axpby(8.0, ref), "gelu_erf", 8.0, s, np.zeros_like(ref), "bf16",
          "4096 full")
