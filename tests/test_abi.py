"""The C ABI on the CPU: the library loads, exports what include/tcm.h
declares, rejects invalid calls with the documented status before touching a
device, and plans the launches it would make.  No compute call runs here."""
import ctypes
import json
import os
import re

import pytest

import tensor_core_matrix_amd as tcm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tcm.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "page_figures.json")

OK, NULLP, BADSHAPE, UNSUP_SHAPE, MISALIGNED, UNSUP_DTYPE, NO_DEVICE, HIP, BADARG = range(9)
A, B, C, SA, SB = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000  # 16-byte aligned stand-ins


def _device_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0  # counts devices without initialising one
    except Exception:  # pragma: no cover
        return False


# The calls here pass stand-in addresses.  Where a device is visible, a call
# that passes validation would launch a kernel on them and fault the GPU, so
# the whole module runs only where no device is.
pytestmark = pytest.mark.skipif(_device_visible(),
                                reason="stand-in pointers must not reach a device")


def test_exports_every_declared_symbol():
    decl = set(re.findall(r"\b(tcm_\w+)\s*\(", open(HEADER).read()))
    assert decl == set(tcm.EXPORTS)
    L = tcm.lib()
    for name in decl:
        assert hasattr(L, name), name


def test_status_strings():
    L = tcm.lib()
    for s in range(9):
        txt = L.tcm_status_string(s).decode()
        assert txt.startswith("TCM_") and ":" in txt
    assert "UNKNOWN" in L.tcm_status_string(99).decode()


def call_plain(a=A, b=B, c=C, M=64, N=64, K=64, dt=tcm.BF16, odt=tcm.BF16):
    return tcm.lib().tcm_gemm_tn(a, b, c, M, N, K, dt, odt, None)


def test_dtype_pairs_rejected():
    for dt, odt in [(tcm.F32, tcm.F32), (tcm.E4M3, tcm.BF16), (tcm.BF16, tcm.F16),
                    (tcm.BF16, tcm.E4M3), (7, tcm.F32)]:
        assert call_plain(dt=dt, odt=odt) == UNSUP_DTYPE
    assert tcm.lib().tcm_gemm_mx_fp8(A, B, SA, SB, C, 64, 64, 64, tcm.F16, None) == UNSUP_DTYPE
    assert tcm.lib().tcm_gemm_mx_fp4(A, B, SA, SB, C, 64, 64, 64, tcm.E4M3, None) == UNSUP_DTYPE


def test_shapes_rejected():
    assert call_plain(M=-1) == BADSHAPE
    assert call_plain(K=-8) == BADSHAPE
    assert call_plain(M=1 << 40, N=1 << 40) == BADSHAPE          # M*N overflows
    assert call_plain(M=1 << 31, K=8) == UNSUP_SHAPE              # beyond 2^30 rows
    assert call_plain(K=(1 << 20) + 8) == UNSUP_SHAPE
    L = tcm.lib()
    assert L.tcm_batched_gemm_tn(A, B, C, -2, 8, 8, 8, tcm.BF16, tcm.F32, None) == BADSHAPE
    assert L.tcm_gemm_mx_fp8(A, B, SA, SB, C, 64, 64, 48, tcm.BF16, None) == UNSUP_SHAPE
    assert L.tcm_gemm_mx_fp4(A, B, SA, SB, C, 64, 64, 48, tcm.BF16, None) == UNSUP_SHAPE
    assert L.tcm_gemm_mx_fp4(A, B, SA, SB, C, -64, 64, 64, tcm.BF16, None) == BADSHAPE


def test_empty_calls_are_no_ops():
    # nothing to write: OK without any pointer or device
    assert call_plain(a=None, b=None, c=None, M=0) == OK
    assert call_plain(a=None, b=None, c=None, N=0) == OK
    assert tcm.lib().tcm_batched_gemm_tn(None, None, None, 0, 8, 8, 8, tcm.BF16,
                                         tcm.F32, None) == OK


def test_null_pointers_rejected():
    assert call_plain(a=None) == NULLP
    assert call_plain(b=None) == NULLP
    assert call_plain(c=None) == NULLP
    L = tcm.lib()
    assert L.tcm_gemm_mx_fp8(A, B, None, SB, C, 64, 64, 64, tcm.BF16, None) == NULLP
    assert L.tcm_gemm_mx_fp8(A, B, SA, None, C, 64, 64, 64, tcm.BF16, None) == NULLP
    assert L.tcm_gemm_mx_fp4(None, B, SA, SB, C, 64, 64, 64, tcm.BF16, None) == NULLP
    assert L.tcm_gemm_mx_fp4(A, B, SA, SB, None, 64, 64, 64, tcm.BF16, None) == NULLP


def test_alignment_rejected():
    assert call_plain(a=A + 2) == MISALIGNED
    assert call_plain(b=B + 8) == MISALIGNED
    assert call_plain(c=C + 4) == MISALIGNED
    assert call_plain(K=60) == MISALIGNED            # 120-byte rows
    L = tcm.lib()
    assert L.tcm_gemm_mx_fp8(A + 1, B, SA, SB, C, 64, 64, 64, tcm.BF16, None) == MISALIGNED
    # scale tensors need no alignment: a valid call gets past validation
    assert L.tcm_gemm_mx_fp8(A, B, SA + 1, SB + 3, C, 64, 64, 64, tcm.BF16, None) in (OK, NO_DEVICE)
    assert L.tcm_gemm_mx_fp4(A, B + 8, SA, SB, C, 64, 64, 64, tcm.BF16, None) == MISALIGNED
    assert L.tcm_gemm_mx_fp4(A, B, SA, SB, C + 2, 64, 64, 64, tcm.F32, None) == MISALIGNED


def test_mxfp6_entry_validation():
    L = tcm.lib()
    f6 = lambda K=64, elem=tcm.E2M3, odt=tcm.BF16, a=A: L.tcm_gemm_mx_fp6(
        a, B, SA, SB, C, 64, 64, K, elem, odt, None)
    assert f6() in (OK, NO_DEVICE)
    assert f6(elem=tcm.E3M2) in (OK, NO_DEVICE)
    assert f6(elem=tcm.E4M3) == UNSUP_DTYPE
    assert f6(odt=tcm.F16) == UNSUP_DTYPE
    assert f6(K=48) == UNSUP_SHAPE          # not whole scale blocks
    assert f6(K=96) == MISALIGNED           # 72-byte rows
    assert f6(a=A + 8) == MISALIGNED
    assert f6(a=None) == NULLP
    p = tcm.plan(8192, 8192, 8192, mx=3)
    assert (p["tile_m"], p["tile_k"], p["stage_bytes"], p["stages"], p["threads"]) == \
        (256, 128, 64 * 1024, 2, 256)


def test_nvfp4_entry_validation():
    L = tcm.lib()
    f = lambda K=64, odt=tcm.BF16, a=A, sa=SA: L.tcm_gemm_nvfp4(a, B, sa, SB, 0.5, 2.0, C, 64, 64,
                                                                K, odt, None)
    assert f() in (OK, NO_DEVICE)
    assert f(odt=tcm.F16) in (OK, NO_DEVICE)
    assert f(odt=tcm.E4M3) == UNSUP_DTYPE
    assert f(K=48) == UNSUP_SHAPE
    assert f(a=A + 8) == MISALIGNED
    assert f(sa=SA + 1) == MISALIGNED       # scales are read two at a time
    assert f(sa=SA + 2) in (OK, NO_DEVICE)
    assert f(a=None) == NULLP


def test_valid_call_without_gpu_reports_no_device():
    assert call_plain() == NO_DEVICE
    assert tcm.lib().tcm_gemm_mx_fp4(A, B, SA, SB, C, 64, 64, 64, tcm.BF16, None) == NO_DEVICE


def call_ex(a=A, b=B, c=SA, o=C, M=64, N=64, K=64, dt=tcm.BF16, cdt=tcm.F32, odt=tcm.F16,
            alpha=1.0, beta=0.5):
    return tcm.lib().tcm_gemm_tn_ex(a, b, c, o, M, N, K, dt, cdt, odt, alpha, beta, None)


def test_epilogue_entry_validation():
    assert call_ex(dt=tcm.F32) == UNSUP_DTYPE
    assert call_ex(odt=tcm.E4M3) == UNSUP_DTYPE
    assert call_ex(cdt=tcm.E8M0) == UNSUP_DTYPE
    assert call_ex(cdt=tcm.E8M0, beta=0.0, c=None) in (OK, NO_DEVICE)  # C unused when beta == 0
    assert call_ex(c=None) == NULLP                                      # beta != 0 needs C
    assert call_ex(o=None) == NULLP
    assert call_ex(M=-1) == BADSHAPE
    assert call_ex(K=(1 << 20) + 8) == UNSUP_SHAPE
    assert call_ex(c=SA + 4) == MISALIGNED
    assert call_ex(K=60) == MISALIGNED
    assert call_ex(a=None, b=None, c=None, o=None, M=0) == OK             # empty: no-op
    assert call_ex() in (OK, NO_DEVICE)


def test_plan_stage_bytes_match_page():
    fig = json.load(open(GOLDEN))["stage_bytes"]
    p = tcm.plan(fig["tile_m"], fig["tile_n"], fig["tile_k"], tcm.BF16, tcm.F32, batch=1024)
    assert (p["tile_m"], p["tile_n"], p["tile_k"]) == (128, 256, 64)
    assert p["stage_bytes"] == fig["stage_KiB"] * 1024
    assert p["lds_bytes"] == p["stages"] * p["stage_bytes"] <= 160 * 1024


def test_plans_of_the_workloads():
    # single tile, one workgroup
    p = tcm.plan(128, 64, 64, tcm.F16, tcm.F32)
    assert p["grid"] == 1 and p["tiles"] == 1 and (p["tile_m"], p["tile_n"]) == (128, 64)
    # 4096^3: one 256 x 256 tile per CU
    p = tcm.plan(4096, 4096, 4096)
    assert (p["tile_m"], p["tile_n"], p["grid"], p["tiles"]) == (256, 256, 256, 256)
    # 8192^3: persistent, four tiles per workgroup
    p = tcm.plan(8192, 8192, 8192)
    assert (p["tile_m"], p["tile_n"], p["grid"], p["tiles"]) == (256, 256, 256, 1024)
    assert p["lds_bytes"] <= 160 * 1024
    # MXFP8 8192^3: 256 x 256 tiles on the 16 x 16 x 128 product, two
    # 128-deep stages (64 KiB each), four waves (variant 31); K not a multiple
    # of 512 (scales not read as 16-byte pieces): eight waves taking turns, a
    # ring of four 64-deep units (32 KiB each; variant 14)
    p = tcm.plan(8192, 8192, 8192, mx=True)
    assert (p["tile_m"], p["tile_k"], p["stage_bytes"], p["stages"], p["threads"], p["kernel"]) == \
        (256, 128, 64 * 1024, 2, 256, 31)
    p = tcm.plan(8192, 8192, 8064, mx=True)
    assert (p["tile_m"], p["tile_k"], p["stage_bytes"], p["stages"], p["threads"], p["kernel"]) == \
        (256, 64, 32 * 1024, 4, 512, 14)
    # MXFP4 8192^3: the 16 x 16 x 128 product, two 256-deep stages of 128-byte
    # rows (64 KiB each), four waves (variant 32); K not a multiple of 512: the
    # ping-pong kernel's ring of four 128-deep 32 KiB units (variant 20)
    p = tcm.plan(8192, 8192, 8192, mx=2)
    assert (p["tile_m"], p["tile_k"], p["stage_bytes"], p["stages"], p["threads"], p["kernel"]) == \
        (256, 256, 64 * 1024, 2, 256, 32)
    p = tcm.plan(8192, 8192, 8064, mx=2)
    assert (p["tile_m"], p["tile_k"], p["stage_bytes"], p["stages"], p["threads"], p["kernel"]) == \
        (256, 128, 32 * 1024, 4, 512, 20)
    # MXFP6 8192^3: the 16 x 16 kernel, 128-deep slices of 96-byte rows kept
    # in 128-byte LDS rows (64 KiB stages, variant 36); K a multiple of 128
    # only (scales read as words): 128-deep units of 96-byte rows (48 KiB) in
    # a ring of three (variant 27); K not a multiple of 128 (scales read byte
    # by byte): the 64-deep kernel's ring of four 24 KiB units (variant 21)
    p = tcm.plan(8192, 8192, 8192, mx=3)
    assert (p["tile_m"], p["tile_k"], p["stage_bytes"], p["stages"], p["kernel"]) == \
        (256, 128, 64 * 1024, 2, 36)
    p = tcm.plan(8192, 8192, 8064, mx=3)
    assert (p["tile_m"], p["tile_k"], p["stage_bytes"], p["stages"], p["kernel"]) == \
        (256, 128, 48 * 1024, 3, 27)
    p = tcm.plan(8192, 8192, 8128, mx=3)
    assert (p["tile_k"], p["stage_bytes"], p["stages"], p["kernel"]) == (64, 24 * 1024, 4, 21)
    # NVFP4 8192^3: the 16 x 16 kernel on 256-deep E2M1 slices, 64 KiB stages
    # (variant 34); K not a multiple of 256: the dequantizing 256 x 256 fp16
    # tile (variant 22); small: 128 x 128
    p = tcm.plan(8192, 8192, 8192, mx=4)
    assert (p["tile_m"], p["tile_n"], p["tile_k"], p["stage_bytes"], p["kernel"]) == \
        (256, 256, 256, 64 * 1024, 34)
    assert tcm.plan(8192, 8192, 8160, mx=4)["kernel"] == 22
    assert tcm.plan(1024, 1024, 1024, mx=4, out_dtype=tcm.F16)["kernel"] == 25
    # MXFP8 with an M- or N-major operand: 256 x 128 x 128 tiles (variant 26),
    # 128 x 128 for problems they would not fill
    # MXFP8 with an M- or N-major operand: the ping-pong kernel's 256 x 256
    # tiles (variant 14) where they fill the CUs, else the 4-wave kernel's
    # 256 x 128 (variant 26) or 128 x 128 tiles
    p = tcm.plan(8192, 8192, 8192, mx=5)
    assert (p["tile_m"], p["tile_n"], p["tile_k"], p["kernel"]) == (256, 256, 64, 14)
    assert tcm.plan(4096, 2048, 4096, mx=5)["kernel"] == 26
    assert tcm.plan(512, 512, 512, mx=5)["kernel"] == 11
    with pytest.raises(tcm.TcmError):
        tcm.plan(64, 64, 64, mx=6)
    with pytest.raises(tcm.TcmError):
        tcm.plan(64, 64, 64, mx=1, out_dtype=tcm.F16)
    # empty problem plans nothing
    assert tcm.plan(0, 8, 8)["grid"] == 0


ROW, COL = tcm.ROW_MAJOR, tcm.COL_MAJOR


def call_gen(a=A, ao=ROW, lda=64, b=B, bo=COL, ldb=64, c=SA, ldc=64, o=C, ldo=64, M=64, N=64,
             K=64, dt=tcm.BF16, cdt=tcm.F32, odt=tcm.F32, alpha=1.0, beta=0.5, op=0):
    return tcm.lib().tcm_gemm(a, ao, lda, b, bo, ldb, c, ldc, o, ldo, M, N, K, dt, cdt, odt,
                              alpha, beta, op, None)


def test_general_entry_validation():
    ok = (OK, NO_DEVICE)
    assert call_gen() in ok
    for ao in (ROW, COL):
        for bo in (ROW, COL):
            assert call_gen(ao=ao, bo=bo) in ok
    # dtypes
    assert call_gen(dt=tcm.F32) == UNSUP_DTYPE
    assert call_gen(odt=tcm.E4M3) == UNSUP_DTYPE
    assert call_gen(cdt=tcm.E8M0) == UNSUP_DTYPE
    assert call_gen(cdt=tcm.E8M0, beta=0.0, c=None, ldc=0) in ok   # C unused when beta == 0
    # orders and leading dimensions
    assert call_gen(ao=2) == BADARG
    assert call_gen(bo=-1) == BADARG
    assert call_gen(op=5) == BADARG
    assert call_gen(op=-1) == BADARG
    for op in range(5):
        assert call_gen(op=op) in ok
    assert call_gen(lda=56, K=64) == BADSHAPE                      # row-major A: lda >= K
    assert call_gen(ao=COL, lda=56, M=64, K=32) == BADSHAPE        # column-major A: lda >= M
    assert call_gen(ao=COL, lda=64, M=64, K=200, ldb=200) in ok    # ... and K is free of lda
    assert call_gen(bo=ROW, ldb=56, N=64) == BADSHAPE              # row-major B: ldb >= N
    assert call_gen(bo=COL, ldb=56, K=64) == BADSHAPE              # column-major B: ldb >= K
    assert call_gen(ldo=63) == BADSHAPE
    assert call_gen(ldc=63) == BADSHAPE
    assert call_gen(ldc=0, beta=0.0, c=None) in ok                 # ldc unused when beta == 0
    assert call_gen(M=-1) == BADSHAPE
    assert call_gen(M=0, a=None, b=None, c=None, o=None) == OK    # empty: no-op
    assert call_gen(M=0, lda=0) == BADSHAPE                        # even then lda >= 1
    # pointers
    assert call_gen(o=None) == NULLP
    assert call_gen(a=None) == NULLP
    assert call_gen(c=None) == NULLP
    # range
    assert call_gen(lda=1 << 22) == UNSUP_SHAPE
    assert call_gen(bo=ROW, ldb=(1 << 21) + 8) == UNSUP_SHAPE
    assert call_gen(lda=1 << 21) in ok
    assert call_gen(ldo=1 << 31) == UNSUP_SHAPE
    # alignment: 16-byte rows and pointers; K % 8 unless both operands are M/N-major
    assert call_gen(lda=68) == MISALIGNED
    assert call_gen(bo=ROW, ldb=100) == MISALIGNED
    assert call_gen(a=A + 8) == MISALIGNED
    assert call_gen(c=SA + 4) == MISALIGNED
    assert call_gen(K=60) == MISALIGNED
    assert call_gen(ao=COL, bo=COL, K=60) == MISALIGNED
    assert call_gen(ao=ROW, bo=ROW, K=60, ldb=64) == MISALIGNED
    assert call_gen(ao=COL, bo=ROW, K=61) in ok
    assert call_gen(ldo=67, ldc=65) in ok                         # Out / C rows are free


def call_mx(a=A, ao=ROW, lda=64, b=B, bo=COL, ldb=64, sa=SA, sb=SB, o=C, ldo=64, M=64, N=64,
            K=64, edt=tcm.E4M3, odt=tcm.BF16):
    return tcm.lib().tcm_gemm_mx(a, ao, lda, b, bo, ldb, sa, sb, o, ldo, M, N, K, edt, odt, None)


def test_mx_general_entry_validation():
    ok = (OK, NO_DEVICE)
    for ao in (ROW, COL):
        for bo in (ROW, COL):
            assert call_mx(ao=ao, bo=bo) in ok
    assert call_mx(odt=tcm.F32) in ok
    # element and output types: E4M3 in, f32 / bf16 out
    assert call_mx(edt=tcm.E2M1) == UNSUP_DTYPE
    assert call_mx(edt=tcm.BF16) == UNSUP_DTYPE
    assert call_mx(odt=tcm.F16) == UNSUP_DTYPE
    # orders and leading dimensions
    assert call_mx(ao=2) == BADARG
    assert call_mx(bo=-1) == BADARG
    assert call_mx(lda=48, K=64) == BADSHAPE                       # row-major A: lda >= K
    assert call_mx(ao=COL, lda=48, M=64, K=32) == BADSHAPE         # column-major A: lda >= M
    assert call_mx(ao=COL, lda=64, M=64, K=256, ldb=256) in ok     # ... and K is free of lda
    assert call_mx(bo=ROW, ldb=48, N=64) == BADSHAPE               # row-major B: ldb >= N
    assert call_mx(ldo=63) == BADSHAPE
    assert call_mx(M=0, a=None, b=None, sa=None, sb=None, o=None) == OK   # empty: no-op
    # pointers
    assert call_mx(o=None) == NULLP
    assert call_mx(sa=None) == NULLP
    assert call_mx(b=None) == NULLP
    # range and shape: K a multiple of 32, ld within 2^21
    assert call_mx(K=48, lda=64, ldb=64) == UNSUP_SHAPE
    assert call_mx(lda=1 << 22) == UNSUP_SHAPE
    assert call_mx(M=-1) == BADSHAPE
    # alignment: rows of whole 16-byte pieces, 16-byte aligned operands
    assert call_mx(lda=72) == MISALIGNED
    assert call_mx(bo=ROW, ldb=72, N=64) == MISALIGNED
    assert call_mx(a=A + 8) == MISALIGNED
    assert call_mx(o=C + 4) == MISALIGNED
    assert call_mx(ldo=67) in ok                                  # Out rows are free


def test_order_ld_of_views():
    import torch
    x = torch.empty(40, 24)
    assert tcm.order_ld(x) == (ROW, 24)
    assert tcm.order_ld(x.T) == (COL, 24)
    assert tcm.order_ld(x[:, :16]) == (ROW, 24)
    assert tcm.order_ld(x[:16, :].T) == (COL, 24)
    with pytest.raises(ValueError):
        tcm.order_ld(x[::2, ::2])


def test_order_ld_of_single_column_and_row_views():
    import torch
    st = torch.empty(1, 304)                 # one stored row of 304
    assert tcm.order_ld(st[:, :300].T) == (COL, 304)   # a 300 x 1 column-major view
    assert tcm.order_ld(st[:, :300]) == (ROW, 304)     # a 1 x 300 row-major view
