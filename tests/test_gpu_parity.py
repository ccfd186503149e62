"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Acceptance per element: |gpu - ref| <= 1e-4 * sum_k |a_ik b_jk|, plus one
bf16 ulp of ref for bf16 output; NaN or Inf always fails.  Exact-input cases
(quarter integers, identity, permutation, all-ones) must match bit for bit.
The measured workloads, at their full sizes and in the launch
configuration the benchmark times, are compared in full in
test_gpu_workloads.py.
"""
import numpy as np
import pytest
import torch

import tensor_core_matrix_amd as tcm
from oracle import oracle as orc
from tensor_core_matrix_amd import inputs as inp

pytestmark = pytest.mark.gpu

DEV = "cuda"
OUT = {"f32": torch.float32, "bf16": torch.bfloat16}
GUARD = 256  # elements of canary on each side of the output


def _guarded(shape, dtype):
    """An output view with NaN canaries before and after it (16-byte aligned)."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * GUARD,), float("nan"), dtype=dtype, device=DEV)
    return buf, buf[GUARD:GUARD + n].view(shape)


def _canaries_intact(buf):
    g = torch.cat([buf[:GUARD], buf[-GUARD:]]).float()
    return bool(torch.isnan(g).all())


def run_plain(a, b, out_dtype, batched=False):
    ad, bd = a.to(DEV), b.to(DEV)
    shape = (a.shape[0], a.shape[1], b.shape[1]) if batched else (a.shape[0], b.shape[0])
    buf, out = _guarded(shape, OUT[out_dtype])
    (tcm.batched_gemm_tn if batched else tcm.gemm_tn)(ad, bd, out)
    torch.cuda.synchronize()
    assert _canaries_intact(buf), "write outside the output"
    return out.cpu()


def run_mx(a, b, sa, sb, out_dtype):
    buf, out = _guarded((a.shape[0], b.shape[0]), OUT[out_dtype])
    tcm.gemm_mx_fp8(a.to(DEV), b.to(DEV), sa.to(DEV), sb.to(DEV), out)
    torch.cuda.synchronize()
    assert _canaries_intact(buf), "write outside the output"
    return out.cpu()


def _np(t):
    return t.double().numpy()


def assert_parity(gpu, ref, s, out_dtype, what=""):
    ok, worst, nbad = orc.check(_np(gpu), ref, s, out_dtype == "bf16")
    assert ok, f"{what}: {nbad} violations, worst err/bound {worst:.3g}"
    return worst


def _dt(name):
    return orc.DTYPE_NAMES[name]


# ------------------------------------------------------------ exact cases
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(128, 64, 64), (16, 8, 32), (512, 384, 256), (1000, 264, 136)])
def test_quarter_integers_exact(dt, shape):
    """Every partial sum is a multiple of 1/16 below 2^24: fp32 output must equal
    the oracle bit for bit, and bf16 output its round-to-nearest-even."""
    M, N, K = shape
    g = inp.generator(100 + M + N + K)
    a = inp.quarter_integers((M, K), g, inp.TORCH_DTYPES[dt])
    b = inp.quarter_integers((N, K), g, inp.TORCH_DTYPES[dt])
    ref, _ = orc.gemm_tn(_dt(dt), inp.raw(a), inp.raw(b))
    out32 = run_plain(a, b, "f32")
    assert np.array_equal(_np(out32), ref)
    out16 = run_plain(a, b, "bf16")
    want = torch.from_numpy(ref).float().to(torch.bfloat16)
    assert torch.equal(out16.view(torch.int16), want.view(torch.int16))


def test_page_warp_example_exact():
    """The 16x8x32 example's inputs (numpy default_rng(0), integers -4..4 over 4)."""
    rng = np.random.default_rng(0)
    a = torch.from_numpy((rng.integers(-4, 5, (16, 32)) / 4).astype("float16"))
    b = torch.from_numpy((rng.integers(-4, 5, (8, 32)) / 4).astype("float16"))
    ref, s = orc.gemm_tn(orc.F16, inp.raw(a), inp.raw(b))
    out = run_plain(a, b, "f32")
    assert np.array_equal(_np(out), ref)
    torch.testing.assert_close(out, torch.from_numpy(ref).float(), rtol=2e-4, atol=2e-4)


def test_identity_and_permutation_exact():
    K, N, M = 256, 320, 192
    g = inp.generator(101)
    b = inp.normal((N, K), g, 1.0, torch.bfloat16)
    out = run_plain(torch.eye(K, dtype=torch.bfloat16), b, "f32")
    assert torch.equal(out, b.float().T.contiguous())
    a = inp.normal((M, K), g, 1.0, torch.bfloat16)
    perm = torch.randperm(K, generator=g)
    p = torch.zeros(K, K, dtype=torch.bfloat16)
    p[torch.arange(K), perm] = 1
    out = run_plain(a, p, "bf16")
    assert torch.equal(out, a[:, perm])


@pytest.mark.parametrize("K", [64, 4096, 8192])
def test_all_ones(K):
    a = torch.ones(256, K, dtype=torch.bfloat16)
    b = torch.ones(512, K, dtype=torch.bfloat16)
    out = run_plain(a, b, "f32")
    assert bool((out == K).all())


# ------------------------------------------------- ragged and edge shapes
SHAPES = [(1, 1, 8), (5, 3, 16), (33, 65, 24), (257, 129, 72), (1000, 777, 520),
          (300, 1000, 1024), (129, 1030, 200)]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("odt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES)
def test_ragged_shapes(dt, odt, shape):
    M, N, K = shape
    g = inp.generator(7 * M + 3 * N + K)
    a = inp.normal((M, K), g, 1.0, inp.TORCH_DTYPES[dt])
    b = inp.normal((N, K), g, 1.0, inp.TORCH_DTYPES[dt])
    ref, s = orc.gemm_tn(_dt(dt), inp.raw(a), inp.raw(b))
    assert_parity(run_plain(a, b, odt), ref, s, odt, f"{dt}->{odt} {shape}")


def test_k_zero_writes_zeros_and_empty_is_noop():
    a = torch.empty(64, 0, dtype=torch.bfloat16)
    b = torch.empty(32, 0, dtype=torch.bfloat16)
    out = run_plain(a, b, "f32")
    assert bool((out == 0).all())
    buf, out = _guarded((0, 16), torch.float32)
    tcm.gemm_tn(torch.empty(0, 64, dtype=torch.bfloat16, device=DEV),
                torch.empty(16, 64, dtype=torch.bfloat16, device=DEV), out)
    torch.cuda.synchronize()
    assert _canaries_intact(buf)


def test_batched_distinct_problems_small():
    g = inp.generator(102)
    a = inp.uniform((37, 40, 64), g, torch.bfloat16)
    b = inp.uniform((37, 72, 64), g, torch.bfloat16)
    ref, s = orc.gemm_tn(orc.BF16, inp.raw(a), inp.raw(b))
    for odt in ("f32", "bf16"):
        assert_parity(run_plain(a, b, odt, batched=True), ref, s, odt, f"batched {odt}")


# -------------------------------------------------------------- MX paths
MX_SHAPES = [(64, 64, 32), (256, 256, 128), (300, 200, 96), (384, 512, 512), (513, 257, 1056)]


@pytest.mark.parametrize("shape", MX_SHAPES)
@pytest.mark.parametrize("odt", ["f32", "bf16"])
def test_mx_shapes(shape, odt):
    M, N, K = shape
    g = inp.generator(M + 5 * N + 11 * K)
    a = inp.e4m3_normal((M, K), g)
    b = inp.e4m3_normal((N, K), g)
    sa = inp.e8m0_scales((M, K // 32), g)
    sb = inp.e8m0_scales((N, K // 32), g)
    ref, s = orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb))
    assert_parity(run_mx(a, b, sa, sb, odt), ref, s, odt, f"mx {shape} {odt}")


def test_mx_unaligned_scale_rows():
    """Scale tensors at odd addresses (byte-wise scale reads)."""
    M, N, K = 256, 256, 256
    g = inp.generator(103)
    a = inp.e4m3_normal((M, K), g)
    b = inp.e4m3_normal((N, K), g)
    sa = inp.e8m0_scales((M, K // 32), g)
    sb = inp.e8m0_scales((N, K // 32), g)
    ref, s = orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb))
    bufa = torch.zeros(sa.numel() + 1, dtype=torch.uint8, device=DEV)
    bufb = torch.zeros(sb.numel() + 3, dtype=torch.uint8, device=DEV)
    va = bufa[1:].view(M, K // 32)
    vb = bufb[3:].view(N, K // 32)
    va.copy_(sa)
    vb.copy_(sb)
    out = torch.empty(M, N, dtype=torch.float32, device=DEV)
    tcm.gemm_mx_fp8(a.to(DEV), b.to(DEV), va, vb, out)
    torch.cuda.synchronize()
    assert_parity(out.cpu(), ref, s, "f32", "mx unaligned scales")


def test_mx_all_ones_closed_form():
    M, N, K = 128, 256, 512
    g = inp.generator(104)
    a = torch.full((M, K), 0x38, dtype=torch.uint8)
    b = torch.full((N, K), 0x38, dtype=torch.uint8)
    sa = inp.e8m0_scales((M, K // 32), g)
    sb = inp.e8m0_scales((N, K // 32), g)
    ea = sa.double() - 127
    eb = sb.double() - 127
    want = (32 * torch.exp2(ea[:, None, :] + eb[None, :, :])).sum(-1)
    out = run_mx(a, b, sa, sb, "f32")
    assert torch.equal(out.double(), want)


def test_mx_unit_scales_match_plain_e4m3():
    M, N, K = 256, 256, 256
    g = inp.generator(105)
    a = inp.e4m3_normal((M, K), g)
    b = inp.e4m3_normal((N, K), g)
    one_a = torch.full((M, K // 32), 127, dtype=torch.uint8)
    one_b = torch.full((N, K // 32), 127, dtype=torch.uint8)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ref, s = orc.entries(orc.E4M3, inp.raw(a), inp.raw(b), ii.ravel(), jj.ravel())
    out = run_mx(a, b, one_a, one_b, "f32")
    assert_parity(out.reshape(-1), ref, s, "f32", "mx unit scales")


def test_repeat_runs_bitwise_identical():
    w = inp.WORKLOADS["bf16_4096"]
    x = inp.make(w)
    a, b = x["A"].to(DEV), x["B"].to(DEV)
    o1 = tcm.gemm_tn(a, b, out_dtype=torch.bfloat16)
    o2 = tcm.gemm_tn(a, b, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


# ------------------------------------------------------ every kernel variant
PLAIN_VARIANTS = [1, 2, 3, 19, 28]
MX_VARIANTS = [11, 14, 31]


@pytest.fixture
def force_variant(monkeypatch):
    def _set(v, max_grid=None):
        monkeypatch.setenv("TCM_FORCE_VARIANT", str(v))
        if max_grid is None:
            monkeypatch.delenv("TCM_MAX_GRID", raising=False)
        else:
            monkeypatch.setenv("TCM_MAX_GRID", str(max_grid))
    return _set


@pytest.mark.parametrize("v", PLAIN_VARIANTS)
def test_each_plain_variant(v, force_variant):
    """Every tile / ring variant, forced: a ragged multi-tile shape with several
    tiles per workgroup, bf16 and fp32 outputs, plus an exact case."""
    force_variant(v)
    M, N, K = 1100, 600, 1000
    g = inp.generator(200 + v)
    a = inp.normal((M, K), g, 1.0, torch.bfloat16)
    b = inp.normal((N, K), g, 1.0, torch.bfloat16)
    ref, s = orc.gemm_tn(orc.BF16, inp.raw(a), inp.raw(b))
    for odt in ("f32", "bf16"):
        assert_parity(run_plain(a, b, odt), ref, s, odt, f"variant {v} {odt}")
    q = inp.quarter_integers((640, 512), g, torch.float16)
    r = inp.quarter_integers((384, 512), g, torch.float16)
    qref, _ = orc.gemm_tn(orc.F16, inp.raw(q), inp.raw(r))
    assert np.array_equal(_np(run_plain(q, r, "f32")), qref)
    # three persistent workgroups: every workgroup walks several tiles, the
    # last of them ragged in M and N
    force_variant(v, max_grid=3)
    for odt in ("f32", "bf16"):
        assert_parity(run_plain(a, b, odt), ref, s, odt, f"variant {v} {odt} grid 3")


@pytest.mark.parametrize("v", MX_VARIANTS)
def test_each_mx_variant(v, force_variant):
    force_variant(v)
    M, N, K = 700, 520, 640
    g = inp.generator(300 + v)
    a = inp.e4m3_normal((M, K), g)
    b = inp.e4m3_normal((N, K), g)
    sa = inp.e8m0_scales((M, K // 32), g)
    sb = inp.e8m0_scales((N, K // 32), g)
    ref, s = orc.gemm_mx(inp.raw(a), inp.raw(b), inp.raw(sa), inp.raw(sb))
    for odt in ("f32", "bf16"):
        assert_parity(run_mx(a, b, sa, sb, odt), ref, s, odt, f"mx variant {v} {odt}")
    # K = 19 scale blocks (byte-wise scale reads, a 32-deep K tail) and three
    # persistent workgroups walking several tiles each
    K2 = 608
    a2 = inp.e4m3_normal((M, K2), g)
    b2 = inp.e4m3_normal((N, K2), g)
    sa2 = inp.e8m0_scales((M, K2 // 32), g)
    sb2 = inp.e8m0_scales((N, K2 // 32), g)
    ref2, s2 = orc.gemm_mx(inp.raw(a2), inp.raw(b2), inp.raw(sa2), inp.raw(sb2))
    force_variant(v, max_grid=3)
    for odt in ("f32", "bf16"):
        assert_parity(run_mx(a2, b2, sa2, sb2, odt), ref2, s2, odt, f"mx variant {v} {odt} K {K2}")
    # K = 1536: scale rows of 48 bytes, read as 16-byte pieces; three chunks
    # of 512 K per tile, several tiles per workgroup
    K3 = 1536
    a3 = inp.e4m3_normal((M, K3), g)
    b3 = inp.e4m3_normal((N, K3), g)
    sa3 = inp.e8m0_scales((M, K3 // 32), g)
    sb3 = inp.e8m0_scales((N, K3 // 32), g)
    ref3, s3 = orc.gemm_mx(inp.raw(a3), inp.raw(b3), inp.raw(sa3), inp.raw(sb3))
    for odt in ("f32", "bf16"):
        assert_parity(run_mx(a3, b3, sa3, sb3, odt), ref3, s3, odt, f"mx variant {v} {odt} K {K3}")


@pytest.mark.parametrize("v", [19, 28])
def test_batched_workload_through_large_tiles(v, force_variant):
    """The batched problems forced through the 256 x 256 persistent kernels
    (half of every tile lies past M = 128)."""
    force_variant(v)
    g = inp.generator(301)
    a = inp.uniform((64, 128, 64), g, torch.bfloat16)
    b = inp.uniform((64, 256, 64), g, torch.bfloat16)
    ref, s = orc.gemm_tn(orc.BF16, inp.raw(a), inp.raw(b))
    assert_parity(run_plain(a, b, "f32", batched=True), ref, s, "f32", "batched via 256x256")
