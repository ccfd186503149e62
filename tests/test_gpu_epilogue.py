"""Parity of the epilogue with a C input, Out = alpha * (A B^T) + beta * C,
with the fp64 oracle through the C ABI.  Acceptance: |alpha| * 1e-4 *
sum_k |a b| for the fp32 sums, 2^-22 of |alpha * sum| + |beta * C| for the
fp32 combine, plus one ulp of a bf16 or fp16 output.  Quarter-integer
operands with power-of-two alpha/beta keep everything exact in fp32, so
those fp32 outputs must match bit for bit."""
import numpy as np
import pytest
import torch

import tensor_core_matrix_amd as tcm
from oracle import oracle as orc
from tensor_core_matrix_amd import inputs as inp

pytestmark = pytest.mark.gpu

DEV = "cuda"
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
GUARD = 256


def guarded(shape, dtype):
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * GUARD,), float("nan"), dtype=dtype, device=DEV)
    return buf, buf[GUARD:GUARD + n].view(shape)


def intact(buf):
    return bool(torch.isnan(torch.cat([buf[:GUARD], buf[-GUARD:]]).float()).all())


def run(a, b, c, alpha, beta, odt):
    buf, out = guarded((a.shape[0], b.shape[0]), TD[odt])
    tcm.gemm_tn_ex(a.to(DEV), b.to(DEV), None if c is None else c.to(DEV), out, alpha, beta)
    torch.cuda.synchronize()
    assert intact(buf), "write outside the output"
    return out.cpu()


def expect(a, b, c, alpha, beta, dt):
    ref, s = orc.gemm_tn(orc.DTYPE_NAMES[dt], inp.raw(a), inp.raw(b))
    if c is None:
        return orc.axpby(alpha, ref), s, np.zeros_like(ref)
    cdt = {torch.float32: orc.F32, torch.bfloat16: orc.BF16, torch.float16: orc.F16}[c.dtype]
    ex = orc.axpby(alpha, ref, beta, inp.raw(c), cdt)
    return ex, s, beta * c.double().numpy()


def check(gpu, ex, alpha, s, bc, odt, what):
    ok, worst, nbad = orc.check_epi(gpu.double().numpy(), ex, alpha, s, bc, odt)
    assert ok, f"{what}: {nbad} violations, worst err/bound {worst:.3g}"


SHAPES = [(1100, 600, 1000), (256, 256, 64), (300, 260, 72), (17, 9, 8), (4096, 512, 256)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("cdt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("odt", ["f32", "bf16", "f16"])
def test_axpby(shape, cdt, odt):
    M, N, K = shape
    g = inp.generator(700 + M + N + K)
    a = inp.normal((M, K), g, 1.0, torch.bfloat16)
    b = inp.normal((N, K), g, 1.0, torch.bfloat16)
    c = inp.normal((M, N), g, 4.0, TD[cdt])
    alpha, beta = 0.75, -1.25
    ex, s, bc = expect(a, b, c, alpha, beta, "bf16")
    check(run(a, b, c, alpha, beta, odt), ex, alpha, s, bc, odt, f"{shape} c {cdt} out {odt}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_beta_zero_without_c_and_fp16_input(dt):
    M, N, K = 700, 330, 200
    g = inp.generator(710)
    a = inp.uniform((M, K), g, TD[dt])
    b = inp.uniform((N, K), g, TD[dt])
    ex, s, bc = expect(a, b, None, -3.0, 0.0, dt)
    check(run(a, b, None, -3.0, 0.0, "f16"), ex, -3.0, s, bc, "f16", f"{dt} beta 0")


def test_in_place_update():
    M, N, K = 520, 700, 128
    g = inp.generator(720)
    a = inp.normal((M, K), g, 1.0, torch.bfloat16)
    b = inp.normal((N, K), g, 1.0, torch.bfloat16)
    c = inp.normal((M, N), g, 2.0, torch.float32)
    ex, s, bc = expect(a, b, c, 2.0, 0.5, "bf16")
    cd = c.to(DEV)
    tcm.gemm_tn_ex(a.to(DEV), b.to(DEV), cd, cd, 2.0, 0.5)  # Out is C
    torch.cuda.synchronize()
    check(cd.cpu(), ex, 2.0, s, bc, "f32", "in place")


def test_exact_quarter_integers():
    M, N, K = 640, 384, 512
    g = inp.generator(730)
    a = inp.quarter_integers((M, K), g, torch.float16)
    b = inp.quarter_integers((N, K), g, torch.float16)
    c = inp.quarter_integers((M, N), g, torch.float32) * 64
    ex, _, _ = expect(a, b, c, 2.0, -0.5, "f16")
    got = run(a, b, c, 2.0, -0.5, "f32").double().numpy()
    assert np.array_equal(got, ex)


def test_large_full_output():
    """4096^3 with a bf16 C, every output against the oracle."""
    M = N = K = 4096
    g = inp.generator(740)
    a = inp.normal((M, K), g, 0.1, torch.bfloat16)
    b = inp.normal((N, K), g, 0.1, torch.bfloat16)
    c = inp.normal((M, N), g, 1.0, torch.bfloat16)
    out = run(a, b, c, 1.5, 0.25, "bf16")
    ref, s = orc.gemm_tn(orc.BF16, inp.raw(a), inp.raw(b))
    ex = orc.axpby(1.5, ref, 0.25, inp.raw(c), orc.BF16)
    check(out, ex, 1.5, s, 0.25 * c.double().numpy(), "bf16", "4096 full")


@pytest.mark.parametrize("variant", [19, 1])
@pytest.mark.parametrize("odt", ["bf16", "f16"])
@pytest.mark.parametrize("grid", [None, 3])
def test_staged_alpha_epilogue(variant, odt, grid, monkeypatch):
    """alpha != 1 without C on the tiles that stage a 16-bit output through
    LDS (256 x 256 and 128 x 256): N a multiple of 8 makes every interior
    tile take the staged form, alpha applied as it is staged, while the
    ragged last tile row (M = 777) keeps the alpha/beta epilogue.  Every
    output against the oracle."""
    monkeypatch.setenv("TCM_FORCE_VARIANT", str(variant))
    if grid:
        monkeypatch.setenv("TCM_MAX_GRID", str(grid))
    M, N, K = 777, 648, 520
    g = inp.generator(760 + variant)
    a = inp.normal((M, K), g, 0.5, torch.bfloat16)
    b = inp.normal((N, K), g, 0.5, torch.bfloat16)
    ex, s, bc = expect(a, b, None, -0.75, 0.0, "bf16")
    check(run(a, b, None, -0.75, 0.0, odt), ex, -0.75, s, bc, odt,
          f"variant {variant} {odt} grid {grid}")
