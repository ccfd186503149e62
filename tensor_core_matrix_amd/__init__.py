"""tensor_core_matrix_amd -- tiled Out = A . B^T on AMD MI355X (gfx950).

A thin ctypes binding over ``libtcm.so`` (C ABI declared in ``include/tcm.h``):
it only marshals torch tensors into pointers, sizes, dtype codes and the
current HIP stream.  Every step of the product runs in the library's HIP
kernels; there is no fallback.  If the library is missing, every call raises.

    gemm_tn(a, b, out=None, out_dtype=None)            a: M x K, b: N x K
    batched_gemm_tn(a, b, out=None, out_dtype=None)    a: B x M x K, b: B x N x K
    gemm_tn_ex(a, b, c=None, out=None, alpha=1.0, beta=0.0, out_dtype=None)
                                                       Out = alpha a . b^T + beta c
    gemm_mx_fp8(a, b, scale_a, scale_b, out=None, out_dtype=torch.bfloat16)
    gemm_mx_fp4(a, b, scale_a, scale_b, out=None, out_dtype=torch.bfloat16)
                                                       a: M x K/2, b: N x K/2 E2M1 pairs
    gemm_mx_fp6(a, b, scale_a, scale_b, out=None, out_dtype=None, elem="e2m3")
                                                       a: M x 3K/4, b: N x 3K/4 packed FP6
    gemm_nvfp4(a, b, scale_a, scale_b, global_a, global_b, out=None, out_dtype=None)
                                                       E2M1 pairs, E4M3 scales per 16
    gemm(a, b, c=None, out=None, alpha=1.0, beta=0.0, out_dtype=None, op="identity")
                                                       Out = op(alpha a . b + beta c), a: M x K
                                                       and b: K x N strided views
    gemm_mx(a, b, scale_a, scale_b, out=None, out_dtype=None)
                                                       MXFP8, a: M x K and b: K x N strided views
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = ["gemm", "gemm_tn", "gemm_tn_ex", "batched_gemm_tn", "gemm_mx_fp8", "gemm_mx_fp4",
           "gemm_mx_fp6", "gemm_nvfp4", "gemm_mx", "order_ld", "plan", "lib", "TcmError",
           "LIB_PATH", "F16", "BF16", "F32", "E4M3", "E8M0", "E2M1", "E2M3", "E3M2", "ROW_MAJOR",
           "COL_MAJOR", "OPS"]

# TCM_LIBRARY names another build of the same library (the host-sanitizer
# build of `python -m tensor_core_matrix_amd.build --sanitize`); by default
# the in-tree libtcm.so.
LIB_PATH = os.environ.get("TCM_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libtcm.so")

# tcm_dtype codes
F16, BF16, F32, E4M3, E8M0, E2M1, E2M3, E3M2 = 0, 1, 2, 3, 4, 5, 6, 7
# tcm_order codes
ROW_MAJOR, COL_MAJOR = 0, 1
# tcm_op codes
OPS = {"identity": 0, "relu": 1, "gelu_tanh": 2, "gelu_erf": 3, "silu": 4}


class TcmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class Plan(ctypes.Structure):
    _fields_ = [("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("tile_k", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("stage_bytes", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("tiles", ctypes.c_int64), ("kernel", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_lock = threading.Lock()
_lib = None
EXPORTS = ("tcm_gemm", "tcm_gemm_tn", "tcm_gemm_tn_ex", "tcm_batched_gemm_tn", "tcm_gemm_mx_fp8",
           "tcm_gemm_mx_fp4", "tcm_gemm_mx_fp6", "tcm_gemm_mx", "tcm_gemm_nvfp4", "tcm_plan_gemm",
           "tcm_status_string")


def lib() -> ctypes.CDLL:
    """The loaded libtcm (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is missing: build it with "
                                  "`python -m tensor_core_matrix_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
            L.tcm_gemm_tn.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp]
            L.tcm_batched_gemm_tn.argtypes = [vp, vp, vp, i64, i64, i64, i64, ci, ci, vp]
            cf = ctypes.c_float
            L.tcm_gemm_tn_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, ci, ci, cf, cf, vp]
            L.tcm_gemm.argtypes = [vp, ci, i64, vp, ci, i64, vp, i64, vp, i64, i64, i64, i64,
                                   ci, ci, ci, cf, cf, ci, vp]
            L.tcm_gemm_mx_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ci, vp]
            L.tcm_gemm_mx_fp4.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ci, vp]
            L.tcm_gemm_mx_fp6.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ci, ci, vp]
            L.tcm_gemm_nvfp4.argtypes = [vp, vp, vp, vp, cf, cf, vp, i64, i64, i64, ci, vp]
            L.tcm_gemm_mx.argtypes = [vp, ci, i64, vp, ci, i64, vp, vp, vp, i64, i64, i64, i64, ci,
                                      ci, vp]
            L.tcm_plan_gemm.argtypes = [i64, i64, i64, i64, ci, ci, ci, ci, ctypes.POINTER(Plan)]
            L.tcm_status_string.argtypes = [ci]
            L.tcm_status_string.restype = ctypes.c_char_p
            for f in ("tcm_gemm", "tcm_gemm_tn", "tcm_gemm_tn_ex", "tcm_batched_gemm_tn", "tcm_gemm_mx_fp8",
                      "tcm_gemm_mx_fp4", "tcm_gemm_mx_fp6", "tcm_gemm_mx", "tcm_gemm_nvfp4",
                      "tcm_plan_gemm"):
                getattr(L, f).restype = ci
            _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().tcm_status_string(status).decode()


def _check(status: int) -> None:
    if status != 0:
        raise TcmError(status, status_string(status))


def _torch():
    import torch
    return torch


def _code(dt) -> int:
    torch = _torch()
    table = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32,
             torch.uint8: E4M3, torch.float8_e4m3fn: E4M3}
    if dt not in table:
        raise TypeError(f"unsupported dtype {dt}")
    return table[dt]


def _ptr(t) -> int:
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def gemm_tn(a, b, out=None, out_dtype=None):
    """Out = a . b^T; a (M, K), b (N, K) float16/bfloat16 CUDA tensors."""
    torch = _torch()
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError(f"K mismatch: {tuple(a.shape)} vs {tuple(b.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=a.device)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be {(M, N)}")
    if a.dtype != b.dtype:
        raise TypeError("a and b must have the same dtype")
    with torch.cuda.device(a.device):
        _check(lib().tcm_gemm_tn(_ptr(a), _ptr(b), _ptr(out), M, N, K, _code(a.dtype),
                                 _code(out.dtype), _stream(a)))
    return out


def batched_gemm_tn(a, b, out=None, out_dtype=None):
    """out[p] = a[p] . b[p]^T; a (batch, M, K), b (batch, N, K)."""
    torch = _torch()
    bt, M, K = a.shape
    if b.shape[0] != bt or b.shape[2] != K:
        raise ValueError(f"shape mismatch: {tuple(a.shape)} vs {tuple(b.shape)}")
    N = b.shape[1]
    if out is None:
        out = torch.empty((bt, M, N), dtype=out_dtype or torch.float32, device=a.device)
    if tuple(out.shape) != (bt, M, N):
        raise ValueError(f"out must be {(bt, M, N)}")
    if a.dtype != b.dtype:
        raise TypeError("a and b must have the same dtype")
    with torch.cuda.device(a.device):
        _check(lib().tcm_batched_gemm_tn(_ptr(a), _ptr(b), _ptr(out), bt, M, N, K,
                                         _code(a.dtype), _code(out.dtype), _stream(a)))
    return out


def gemm_mx_fp8(a, b, scale_a, scale_b, out=None, out_dtype=None):
    """MXFP8 Out = (a * scale_a) . (b * scale_b)^T.  a (M, K), b (N, K) E4M3 bytes
    (uint8 or float8_e4m3fn); scale_a (M, K/32), scale_b (N, K/32) E8M0 bytes."""
    torch = _torch()
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("K mismatch")
    if K % 32 or tuple(scale_a.shape) != (M, K // 32) or tuple(scale_b.shape) != (N, K // 32):
        raise ValueError("scale tensors must be (rows, K/32) with K a multiple of 32")
    for t in (a, b):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError("MX elements must be uint8 or float8_e4m3fn")
    for t in (scale_a, scale_b):
        if t.dtype not in (torch.uint8, torch.float8_e8m0fnu):
            raise TypeError("MX scales must be uint8 or float8_e8m0fnu")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=a.device)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be {(M, N)}")
    with torch.cuda.device(a.device):
        _check(lib().tcm_gemm_mx_fp8(_ptr(a), _ptr(b), _ptr(scale_a), _ptr(scale_b), _ptr(out),
                                     M, N, K, _code(out.dtype), _stream(a)))
    return out


def gemm_tn_ex(a, b, c=None, out=None, alpha=1.0, beta=0.0, out_dtype=None):
    """Out = alpha * a . b^T + beta * c; a (M, K), b (N, K) float16/bfloat16;
    c (M, N) float16/bfloat16/float32 or None (then beta must be 0); out
    float16/bfloat16/float32 and may be c itself."""
    torch = _torch()
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K or b.dtype != a.dtype:
        raise ValueError("a and b must share K and dtype")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=a.device)
    if tuple(out.shape) != (M, N) or (c is not None and tuple(c.shape) != (M, N)):
        raise ValueError(f"out and c must be {(M, N)}")
    if c is None and beta != 0.0:
        raise ValueError("beta != 0 needs c")
    codes = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}
    for t in (out,) + ((c,) if c is not None else ()):
        if t.dtype not in codes:
            raise TypeError(f"unsupported dtype {t.dtype}")
    with torch.cuda.device(a.device):
        _check(lib().tcm_gemm_tn_ex(_ptr(a), _ptr(b), None if c is None else _ptr(c), _ptr(out),
                                    M, N, K, _code(a.dtype), codes[c.dtype] if c is not None else F32,
                                    codes[out.dtype], float(alpha), float(beta), _stream(a)))
    return out


def gemm_mx_fp4(a, b, scale_a, scale_b, out=None, out_dtype=None):
    """MXFP4 Out = (a * scale_a) . (b * scale_b)^T.  a (M, K/2), b (N, K/2) uint8
    holding two E2M1 elements each (element 2t in the low four bits of byte t);
    scale_a (M, K/32), scale_b (N, K/32) E8M0 bytes."""
    torch = _torch()
    M, KH = a.shape
    N = b.shape[0]
    K = 2 * KH
    if b.shape[1] != KH:
        raise ValueError("K mismatch")
    if K % 32 or tuple(scale_a.shape) != (M, K // 32) or tuple(scale_b.shape) != (N, K // 32):
        raise ValueError("scale tensors must be (rows, K/32) with K a multiple of 32")
    for t in (a, b):
        if t.dtype != torch.uint8:
            raise TypeError("MXFP4 elements must be uint8 pairs")
    for t in (scale_a, scale_b):
        if t.dtype not in (torch.uint8, torch.float8_e8m0fnu):
            raise TypeError("MX scales must be uint8 or float8_e8m0fnu")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=a.device)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be {(M, N)}")
    with torch.cuda.device(a.device):
        _check(lib().tcm_gemm_mx_fp4(_ptr(a), _ptr(b), _ptr(scale_a), _ptr(scale_b), _ptr(out),
                                     M, N, K, _code(out.dtype), _stream(a)))
    return out


def order_ld(t) -> tuple[int, int]:
    """(tcm_order, leading dimension) of a 2-D tensor view whose rows or
    columns are contiguous (unit stride along dimension 1 or 0)."""
    r, c = t.shape
    s0, s1 = t.stride()
    if s1 == 1 and (s0 >= c or r <= 1):
        return ROW_MAJOR, s0 if r > 1 else max(s0, c)
    if s0 == 1 and (s1 >= r or c <= 1):
        return COL_MAJOR, s1 if c > 1 else max(s1, r)
    raise ValueError(f"no unit stride: shape {tuple(t.shape)}, strides {t.stride()}")


def gemm(a, b, c=None, out=None, alpha=1.0, beta=0.0, out_dtype=None, op="identity"):
    """Out = op(alpha * a . b + beta * c) for 2-D views: a (M, K) and b (K, N)
    float16/bfloat16 with rows or columns contiguous (transposed views and
    slices of larger tensors are taken as they are, by their strides); c and
    out (M, N) float16/bfloat16/float32 with contiguous rows; out may be c.
    op: "identity", "relu", "gelu_tanh", "gelu_erf" or "silu"."""
    torch = _torch()
    M, K = a.shape
    K2, N = b.shape
    if K2 != K or b.dtype != a.dtype:
        raise ValueError("a (M, K) and b (K, N) must share K and dtype")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=a.device)
    if tuple(out.shape) != (M, N) or (c is not None and tuple(c.shape) != (M, N)):
        raise ValueError(f"out and c must be {(M, N)}")
    if c is None and beta != 0.0:
        raise ValueError("beta != 0 needs c")
    codes = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}
    for t in (out,) + ((c,) if c is not None else ()):
        if t.dtype not in codes:
            raise TypeError(f"unsupported dtype {t.dtype}")
    ao, lda = order_ld(a)
    bo, ldb = order_ld(b)
    oo, ldo = order_ld(out)
    co, ldc = order_ld(c) if c is not None else (ROW_MAJOR, N)
    if oo != ROW_MAJOR or co != ROW_MAJOR:
        raise ValueError("out and c need contiguous rows")
    with torch.cuda.device(a.device):
        _check(lib().tcm_gemm(a.data_ptr(), ao, lda, b.data_ptr(), bo, ldb,
                              None if c is None else c.data_ptr(), ldc, out.data_ptr(), ldo,
                              M, N, K, _code(a.dtype), codes[c.dtype] if c is not None else F32,
                              codes[out.dtype], float(alpha), float(beta), OPS[op], _stream(a)))
    return out


def gemm_mx(a, b, scale_a, scale_b, out=None, out_dtype=None):
    """MXFP8 Out = (a * scale_a) . (b * scale_b) for 2-D views: a (M, K) and
    b (K, N) of E4M3 elements (float8_e4m3fn or uint8) with rows or columns
    contiguous (transposed views and slices of larger tensors are taken by
    their strides); scale_a (M, K/32) and scale_b (N, K/32) E8M0 bytes, one
    per 32 K values of a row of a and of a column of b; out (M, N)
    float32/bfloat16 with contiguous rows."""
    torch = _torch()
    M, K = a.shape
    K2, N = b.shape
    if K2 != K:
        raise ValueError("a (M, K) and b (K, N) must share K")
    if K % 32 or tuple(scale_a.shape) != (M, K // 32) or tuple(scale_b.shape) != (N, K // 32):
        raise ValueError("scale tensors must be (M, K/32) and (N, K/32) with K a multiple of 32")
    for t in (a, b):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError("MXFP8 elements must be float8_e4m3fn or uint8")
    for t in (scale_a, scale_b):
        if t.dtype not in (torch.uint8, torch.float8_e8m0fnu) or not t.is_contiguous():
            raise TypeError("MX scales must be contiguous uint8 or float8_e8m0fnu")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=a.device)
    codes = {torch.bfloat16: BF16, torch.float32: F32}
    if tuple(out.shape) != (M, N) or out.dtype not in codes:
        raise ValueError(f"out must be {(M, N)} float32 or bfloat16")
    ao, lda = order_ld(a)
    bo, ldb = order_ld(b)
    oo, ldo = order_ld(out)
    if oo != ROW_MAJOR:
        raise ValueError("out needs contiguous rows")
    with torch.cuda.device(a.device):
        _check(lib().tcm_gemm_mx(a.data_ptr(), ao, lda, b.data_ptr(), bo, ldb, scale_a.data_ptr(),
                                 scale_b.data_ptr(), out.data_ptr(), ldo, M, N, K, E4M3,
                                 codes[out.dtype], _stream(a)))
    return out


def gemm_mx_fp6(a, b, scale_a, scale_b, out=None, out_dtype=None, elem="e2m3"):
    """MXFP6 Out = (a * scale_a) . (b * scale_b)^T.  a (M, 3K/4), b (N, 3K/4)
    uint8 holding packed 6-bit codes (element t of a row in bits 6t .. 6t+5);
    scale_a (M, K/32), scale_b (N, K/32) E8M0 bytes; elem "e2m3" or "e3m2"."""
    torch = _torch()
    M, KB = a.shape
    N = b.shape[0]
    if KB % 3 or b.shape[1] != KB:
        raise ValueError("packed FP6 rows of equal length, whole three-byte groups")
    K = KB // 3 * 4
    if K % 32 or tuple(scale_a.shape) != (M, K // 32) or tuple(scale_b.shape) != (N, K // 32):
        raise ValueError("scale tensors must be (rows, K/32) with K a multiple of 32")
    for t in (a, b):
        if t.dtype != torch.uint8:
            raise TypeError("MXFP6 codes must be packed in uint8")
    for t in (scale_a, scale_b):
        if t.dtype not in (torch.uint8, torch.float8_e8m0fnu):
            raise TypeError("MX scales must be uint8 or float8_e8m0fnu")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=a.device)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be {(M, N)}")
    code = {"e2m3": E2M3, "e3m2": E3M2}[elem]
    with torch.cuda.device(a.device):
        _check(lib().tcm_gemm_mx_fp6(_ptr(a), _ptr(b), _ptr(scale_a), _ptr(scale_b), _ptr(out),
                                     M, N, K, code, _code(out.dtype), _stream(a)))
    return out


def gemm_nvfp4(a, b, scale_a, scale_b, global_a=1.0, global_b=1.0, out=None, out_dtype=None):
    """NVFP4 Out = global_a global_b (a * scale_a) . (b * scale_b)^T.  a (M, K/2),
    b (N, K/2) uint8 E2M1 pairs (element 2t in the low four bits of byte t);
    scale_a (M, K/16), scale_b (N, K/16) E4M3 block scales (uint8 or
    float8_e4m3fn); global_a, global_b the fp32 per-tensor scales."""
    torch = _torch()
    M, KH = a.shape
    N = b.shape[0]
    K = 2 * KH
    if b.shape[1] != KH:
        raise ValueError("K mismatch")
    if K % 32 or tuple(scale_a.shape) != (M, K // 16) or tuple(scale_b.shape) != (N, K // 16):
        raise ValueError("scale tensors must be (rows, K/16) with K a multiple of 32")
    for t in (a, b):
        if t.dtype != torch.uint8:
            raise TypeError("NVFP4 elements must be uint8 pairs")
    for t in (scale_a, scale_b):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError("NVFP4 scales must be uint8 or float8_e4m3fn")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=a.device)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be {(M, N)}")
    codes = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}
    with torch.cuda.device(a.device):
        _check(lib().tcm_gemm_nvfp4(_ptr(a), _ptr(b), _ptr(scale_a), _ptr(scale_b),
                                    float(global_a), float(global_b), _ptr(out), M, N, K,
                                    codes[out.dtype], _stream(a)))
    return out


def plan(M, N, K, dtype=BF16, out_dtype=BF16, batch=1, mx=False, num_cus=256) -> dict:
    """The launch a call would make (tile, ring depth, LDS bytes, grid).  mx:
    False (or 0) plain, True (or 1) MXFP8, 2 MXFP4, 3 MXFP6, 4 NVFP4, 5 MXFP8
    with an M- or N-major operand (gemm_mx)."""
    p = Plan()
    _check(lib().tcm_plan_gemm(batch, M, N, K, dtype, out_dtype, int(mx), num_cus,
                               ctypes.byref(p)))
    return p.as_dict()
