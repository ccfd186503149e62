"""Plain fp64 CPU oracle for Out = A . B^T (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product library never does: the
oracle shares no code with the HIP path, and the HIP path never falls back to
it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, sequential sums over K,
threads over output rows).  This wrapper builds it with gcc, passes raw input
storage through ctypes, and holds the elementwise comparison rule:

    |gpu - ref| <= 1e-4 * sum_k |a_ik * b_jk|  (+ one bf16 ulp of ref when the
                                                 output is bf16)

The rule states the accuracy expected of an fp32-accumulating product whose
element products are exact ("Blackwell Tensor Cores", The Accumulator's
Lifetime: float16 products accumulated in float32).  Its bf16 ulp term covers
the single rounding of the fp32 result to a bf16 output.

``gemm_ld`` / ``entries_ld`` take the operands in either arrangement
(row-major or column-major A and B of Out = A . B) with leading dimensions,
as the cuBLASDx Blackwell card's host side declares global operands.

Inputs are numpy arrays holding the raw storage of the operands:
uint16 for float16 / bfloat16 bit patterns, uint8 for E4M3 and E8M0 bytes,
uint8 for E2M1 pairs (two elements per byte, the even element in the low four
bits, so an M x K operand is stored M x K/2), float32 for float32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

F16, BF16, F32, E4M3, E8M0, E2M1, E2M3, E3M2 = 0, 1, 2, 3, 4, 5, 6, 7
DTYPE_NAMES = {"f16": F16, "bf16": BF16, "f32": F32, "e4m3": E4M3, "e8m0": E8M0, "e2m1": E2M1,
               "e2m3": E2M3, "e3m2": E3M2}
# elements per storage byte-group: (elements, bytes) of the packed formats
_PACK = {E2M1: (2, 1), E2M3: (4, 3), E3M2: (4, 3)}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_SAN_LIB = os.path.join(_HERE, "liboracle_san.so")
# ORACLE_LIBRARY names another build of oracle.c (the sanitizer build below)
_USE = os.environ.get("ORACLE_LIBRARY")
_lock = threading.Lock()
_lib = None


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile oracle.c into liboracle.so beside it (gcc, -O2, no fast-math so
    the fp64 sums keep their sequential order).  sanitize: liboracle_san.so,
    the same with AddressSanitizer and UndefinedBehaviorSanitizer, for CPU
    runs of the oracle's tests (load it with ORACLE_LIBRARY and libasan
    preloaded)."""
    lib = _SAN_LIB if sanitize else _LIB
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
        tmp = lib + ".tmp%d" % os.getpid()
        san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g"] if sanitize else []
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
             "-fno-fast-math", "-ffp-contract=off", *san, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(_USE) if _USE else ctypes.CDLL(build(force=False))
            i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
            lib.oracle_decode.argtypes = [ctypes.c_int, vp, i64, dp]
            lib.oracle_gemm_tn.argtypes = [ctypes.c_int, vp, vp, i64, i64, i64, i64, dp, dp,
                                           ctypes.c_int]
            lib.oracle_gemm_mx.argtypes = [vp, vp, vp, vp, i64, i64, i64, dp, dp, ctypes.c_int]
            lib.oracle_gemm_mx_typed.argtypes = [ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, dp,
                                                 dp, ctypes.c_int]
            lib.oracle_axpby.argtypes = [i64, ctypes.c_double, dp, ctypes.c_double, ctypes.c_int,
                                         vp, dp]
            lib.oracle_entries.argtypes = [ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, vp, vp,
                                           vp, i64, dp, dp]
            ci = ctypes.c_int
            lib.oracle_gemm_ld.argtypes = [ci, vp, ci, i64, vp, ci, i64, i64, i64, i64, dp, dp,
                                           ci]
            lib.oracle_entries_ld.argtypes = [ci, vp, ci, i64, vp, ci, i64, i64, i64, i64, vp,
                                              vp, i64, dp, dp]
            lib.oracle_apply_op.argtypes = [i64, ci, dp, dp]
            lib.oracle_gemm_mx_ld.argtypes = [vp, ci, i64, vp, ci, i64, vp, vp, i64, i64, i64, dp,
                                              dp, ci]
            lib.oracle_entries_mx_ld.argtypes = [vp, ci, i64, vp, ci, i64, vp, vp, i64, i64, i64,
                                                 vp, vp, i64, dp, dp]
            cd = ctypes.c_double
            lib.oracle_gemm_nvfp4.argtypes = [vp, vp, vp, vp, cd, cd, i64, i64, i64, dp, dp, ci]
            lib.oracle_entries_nvfp4.argtypes = [vp, vp, vp, vp, cd, cd, i64, i64, i64, vp, vp, i64,
                                                 dp, dp]
            for f in (lib.oracle_decode, lib.oracle_gemm_tn, lib.oracle_gemm_mx,
                      lib.oracle_gemm_mx_typed, lib.oracle_entries, lib.oracle_axpby,
                      lib.oracle_gemm_ld, lib.oracle_entries_ld, lib.oracle_apply_op,
                      lib.oracle_gemm_nvfp4, lib.oracle_entries_nvfp4, lib.oracle_gemm_mx_ld,
                      lib.oracle_entries_mx_ld):
                f.restype = ctypes.c_int
            _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


_STORAGE = {F16: np.uint16, BF16: np.uint16, F32: np.float32, E4M3: np.uint8, E8M0: np.uint8,
            E2M1: np.uint8, E2M3: np.uint8, E3M2: np.uint8}


def _raw(x: np.ndarray, dtype: int) -> np.ndarray:
    want = _STORAGE[dtype]
    x = np.ascontiguousarray(x)
    if x.dtype.itemsize != np.dtype(want).itemsize:
        raise TypeError(f"storage of dtype {dtype} must be {np.dtype(want)}, got {x.dtype}")
    return x


def _ptr(x):
    return None if x is None else x.ctypes.data


def decode(dtype: int, raw: np.ndarray) -> np.ndarray:
    """Exact fp64 values of stored elements (format definitions, see oracle.c).
    E2M1 storage of shape (..., n) decodes to shape (..., 2 n), FP6 storage
    (E2M3, E3M2) of shape (..., 3 n) to shape (..., 4 n)."""
    raw = _raw(raw, dtype)
    if dtype in _PACK:
        e, b = _PACK[dtype]
        if raw.shape[-1] % b:
            raise ValueError("packed rows must be whole byte groups")
        shape = raw.shape[:-1] + (raw.shape[-1] // b * e,)
    else:
        shape = raw.shape
    out = np.empty(shape, dtype=np.float64)
    rc = _load().oracle_decode(dtype, _ptr(raw), out.size, _ptr(out))
    if rc:
        raise ValueError(f"oracle_decode failed ({rc})")
    return out


def gemm_tn(dtype: int, a: np.ndarray, b: np.ndarray, nthreads: int | None = None):
    """ref, abssum for Out = A . B^T.  a: [batch,] M x K, b: [batch,] N x K raw
    storage.  Returns fp64 arrays of shape [batch,] M x N."""
    a, b = _raw(a, dtype), _raw(b, dtype)
    batched = a.ndim == 3
    if not batched:
        a, b = a[None], b[None]
    if a.ndim != 3 or b.ndim != 3 or a.shape[0] != b.shape[0] or a.shape[2] != b.shape[2]:
        raise ValueError(f"bad shapes {a.shape} {b.shape}")
    bt, M, K = a.shape
    N = b.shape[1]
    ref = np.empty((bt, M, N), np.float64)
    s = np.empty((bt, M, N), np.float64)
    rc = _load().oracle_gemm_tn(dtype, _ptr(a), _ptr(b), bt, M, N, K, _ptr(ref), _ptr(s),
                                nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_gemm_tn failed ({rc})")
    return (ref, s) if batched else (ref[0], s[0])


def gemm_mx(a: np.ndarray, b: np.ndarray, sa: np.ndarray, sb: np.ndarray,
            nthreads: int | None = None, dtype: int = E4M3):
    """ref, abssum for the MX block-scaled product: a M x K, b N x K elements of
    `dtype` (E4M3 bytes; E2M1 pairs stored M x K/2 and N x K/2; FP6 (E2M3,
    E3M2) stored M x 3K/4 and N x 3K/4); sa M x K/32, sb N x K/32 E8M0 bytes."""
    a, b, sa, sb = _raw(a, dtype), _raw(b, dtype), _raw(sa, E8M0), _raw(sb, E8M0)
    M = a.shape[0]
    N = b.shape[0]
    e, by = _PACK.get(dtype, (1, 1))
    K = a.shape[1] // by * e
    if b.shape[1] != a.shape[1] or K % 32 or sa.shape != (M, K // 32) or sb.shape != (N, K // 32):
        raise ValueError("bad MX shapes")
    ref = np.empty((M, N), np.float64)
    s = np.empty((M, N), np.float64)
    rc = _load().oracle_gemm_mx_typed(dtype, _ptr(a), _ptr(b), _ptr(sa), _ptr(sb), M, N, K,
                                      _ptr(ref), _ptr(s), nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_gemm_mx failed ({rc})")
    return ref, s


def _nv4_args(a, b, sa, sb):
    a, b = _raw(a, E2M1), _raw(b, E2M1)
    sa, sb = _raw(sa, E4M3), _raw(sb, E4M3)
    M, N, K = a.shape[0], b.shape[0], a.shape[1] * 2
    if b.shape[1] * 2 != K or K % 16 or sa.shape != (M, K // 16) or sb.shape != (N, K // 16):
        raise ValueError("bad NVFP4 shapes")
    return a, b, sa, sb, M, N, K


def gemm_nvfp4(a, b, sa, sb, ga: float, gb: float, nthreads: int | None = None):
    """ref, abssum for the NVFP4 product (see oracle.c): a M x K/2, b N x K/2
    E2M1 pairs; sa M x K/16, sb N x K/16 E4M3 bytes; ga, gb the per-tensor
    fp32 scales."""
    a, b, sa, sb, M, N, K = _nv4_args(a, b, sa, sb)
    ref = np.empty((M, N), np.float64)
    s = np.empty((M, N), np.float64)
    rc = _load().oracle_gemm_nvfp4(_ptr(a), _ptr(b), _ptr(sa), _ptr(sb), float(ga), float(gb), M,
                                   N, K, _ptr(ref), _ptr(s), nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_gemm_nvfp4 failed ({rc})")
    return ref, s


def entries_nvfp4(a, b, sa, sb, ga: float, gb: float, ii, jj):
    """ref, abssum at outputs (ii[t], jj[t]) of the NVFP4 product."""
    a, b, sa, sb, M, N, K = _nv4_args(a, b, sa, sb)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    ref = np.empty(ii.size, np.float64)
    s = np.empty(ii.size, np.float64)
    rc = _load().oracle_entries_nvfp4(_ptr(a), _ptr(b), _ptr(sa), _ptr(sb), float(ga), float(gb),
                                      M, N, K, _ptr(ii), _ptr(jj), ii.size, _ptr(ref), _ptr(s))
    if rc:
        raise ValueError(f"oracle_entries_nvfp4 failed ({rc})")
    return ref, s


def entries(dtype: int, a: np.ndarray, b: np.ndarray, ii, jj, bb=None, sa=None, sb=None):
    """ref, abssum at selected outputs (ii[t], jj[t]) [of problem bb[t]], each
    computed one by one from the definition; for problems too big to do whole."""
    a, b = _raw(a, dtype), _raw(b, dtype)
    if a.ndim == 2:
        a3, b3 = a[None], b[None]
    else:
        a3, b3 = a, b
    _, M, K = a3.shape
    if dtype in _PACK:
        K = K // _PACK[dtype][1] * _PACK[dtype][0]
    N = b3.shape[1]
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    bbv = None if bb is None else np.ascontiguousarray(bb, dtype=np.int64)
    if sa is not None:
        sa, sb = _raw(sa, E8M0), _raw(sb, E8M0)
    n = ii.size
    ref = np.empty(n, np.float64)
    s = np.empty(n, np.float64)
    rc = _load().oracle_entries(dtype, _ptr(a3), _ptr(b3), _ptr(sa), _ptr(sb), M, N, K,
                                _ptr(bbv), _ptr(ii), _ptr(jj), n, _ptr(ref), _ptr(s))
    if rc:
        raise ValueError(f"oracle_entries failed ({rc})")
    return ref, s


ROW_MAJOR, COL_MAJOR = 0, 1


def storage_elems(order: int, ld: int, rows: int, cols: int) -> int:
    """Elements a rows x cols matrix of the given order and leading dimension
    spans in storage (0 when it is empty)."""
    if rows == 0 or cols == 0:
        return 0
    return (rows - 1) * ld + cols if order == ROW_MAJOR else (cols - 1) * ld + rows


def _ld_args(dtype, a, a_order, lda, b, b_order, ldb, M, N, K):
    a = _raw(a, dtype).reshape(-1)
    b = _raw(b, dtype).reshape(-1)
    if a.size < storage_elems(a_order, lda, M, K) or b.size < storage_elems(b_order, ldb, K, N):
        raise ValueError("operand storage smaller than its shape and leading dimension need")
    return a, b


def gemm_ld(dtype: int, a: np.ndarray, a_order: int, lda: int, b: np.ndarray, b_order: int,
            ldb: int, M: int, N: int, K: int, nthreads: int | None = None):
    """ref, abssum (fp64, M x N) of Out = A . B with A the M x K matrix and B
    the K x N matrix, each stored row-major or column-major (ROW_MAJOR /
    COL_MAJOR) with leading dimension lda / ldb in elements (see oracle.c).
    a and b are raw storage, any shape, read flat."""
    a, b = _ld_args(dtype, a, a_order, lda, b, b_order, ldb, M, N, K)
    ref = np.empty((M, N), np.float64)
    s = np.empty((M, N), np.float64)
    rc = _load().oracle_gemm_ld(dtype, _ptr(a), a_order, lda, _ptr(b), b_order, ldb, M, N, K,
                                _ptr(ref), _ptr(s), nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_gemm_ld failed ({rc})")
    return ref, s


def entries_ld(dtype: int, a, a_order: int, lda: int, b, b_order: int, ldb: int, M: int, N: int,
               K: int, ii, jj):
    """ref, abssum at outputs (ii[t], jj[t]) of the gemm_ld product, each from
    the definition, for problems too big to do whole."""
    a, b = _ld_args(dtype, a, a_order, lda, b, b_order, ldb, M, N, K)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    ref = np.empty(ii.size, np.float64)
    s = np.empty(ii.size, np.float64)
    rc = _load().oracle_entries_ld(dtype, _ptr(a), a_order, lda, _ptr(b), b_order, ldb, M, N, K,
                                   _ptr(ii), _ptr(jj), ii.size, _ptr(ref), _ptr(s))
    if rc:
        raise ValueError(f"oracle_entries_ld failed ({rc})")
    return ref, s


def _mx_ld_args(a, a_order, lda, b, b_order, ldb, sa, sb, M, N, K):
    a, b = _ld_args(E4M3, a, a_order, lda, b, b_order, ldb, M, N, K)
    sa, sb = _raw(sa, E8M0), _raw(sb, E8M0)
    if K % 32 or sa.shape != (M, K // 32) or sb.shape != (N, K // 32):
        raise ValueError("MX scales must be M x K/32 and N x K/32 with K a multiple of 32")
    return a, b, sa, sb


def gemm_mx_ld(a, a_order: int, lda: int, b, b_order: int, ldb: int, sa, sb, M: int, N: int,
               K: int, nthreads: int | None = None):
    """ref, abssum of the MXFP8 product with A (M x K) and B (K x N) E4M3
    elements in either arrangement with leading dimensions (raw storage, read
    flat), sa M x K/32 and sb N x K/32 E8M0 scales (see oracle.c)."""
    a, b, sa, sb = _mx_ld_args(a, a_order, lda, b, b_order, ldb, sa, sb, M, N, K)
    ref = np.empty((M, N), np.float64)
    s = np.empty((M, N), np.float64)
    rc = _load().oracle_gemm_mx_ld(_ptr(a), a_order, lda, _ptr(b), b_order, ldb, _ptr(sa),
                                   _ptr(sb), M, N, K, _ptr(ref), _ptr(s),
                                   nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_gemm_mx_ld failed ({rc})")
    return ref, s


def entries_mx_ld(a, a_order: int, lda: int, b, b_order: int, ldb: int, sa, sb, M: int, N: int,
                  K: int, ii, jj):
    """ref, abssum at outputs (ii[t], jj[t]) of the gemm_mx_ld product."""
    a, b, sa, sb = _mx_ld_args(a, a_order, lda, b, b_order, ldb, sa, sb, M, N, K)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    ref = np.empty(ii.size, np.float64)
    s = np.empty(ii.size, np.float64)
    rc = _load().oracle_entries_mx_ld(_ptr(a), a_order, lda, _ptr(b), b_order, ldb, _ptr(sa),
                                      _ptr(sb), M, N, K, _ptr(ii), _ptr(jj), ii.size, _ptr(ref),
                                      _ptr(s))
    if rc:
        raise ValueError(f"oracle_entries_mx_ld failed ({rc})")
    return ref, s


def axpby(alpha: float, ref: np.ndarray, beta: float = 0.0, c: np.ndarray | None = None,
          c_dtype: int = F32) -> np.ndarray:
    """alpha * ref + beta * C in fp64 (C given as raw storage of c_dtype, same
    shape as ref; may be None when beta == 0)."""
    ref = np.ascontiguousarray(ref, np.float64)
    out = np.empty_like(ref)
    cr = None if c is None else _raw(c, c_dtype)
    if cr is not None and cr.shape != ref.shape:
        raise ValueError("C shape must equal the output shape")
    rc = _load().oracle_axpby(ref.size, float(alpha), _ptr(ref), float(beta), c_dtype,
                              _ptr(cr), _ptr(out))
    if rc:
        raise ValueError(f"oracle_axpby failed ({rc})")
    return out


OPS = {"identity": 0, "relu": 1, "gelu_tanh": 2, "gelu_erf": 3, "silu": 4}
# Largest |op'(x)| over all x: 1 for identity and relu; silu's maximum is
# 1.0998 (at x = 2.3994), both gelu forms' 1.1289 (near x = 1.41).
OP_LIPSCHITZ = {0: 1.0, 1: 1.0, 2: 1.13, 3: 1.13, 4: 1.1}


def apply_op(op: int, x: np.ndarray) -> np.ndarray:
    """The epilogue's per-element operation in fp64 (see oracle.c)."""
    x = np.ascontiguousarray(x, np.float64)
    out = np.empty_like(x)
    rc = _load().oracle_apply_op(x.size, int(op), _ptr(x), _ptr(out))
    if rc:
        raise ValueError(f"oracle_apply_op failed ({rc})")
    return out


# ----------------------------------------------------------------------------
# Comparison rule
# ----------------------------------------------------------------------------
REL_TOL = 1e-4


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x|: 2^(max(floor(log2|x|), -126) - 7),
    and the subnormal spacing 2^-133 at zero (bfloat16 keeps 7 stored mantissa
    bits and binary32's exponent range)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.full(x.shape, -126.0)
    nz = x > 0
    e[nz] = np.maximum(np.floor(np.log2(x[nz])), -126.0)
    return np.exp2(e - 7.0)


def ulp_f16(x: np.ndarray) -> np.ndarray:
    """Spacing of IEEE binary16 numbers at |x|: 2^(max(floor(log2|x|), -14) - 10)
    (10 stored mantissa bits, smallest normal exponent -14, subnormal spacing
    2^-24)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.full(x.shape, -14.0)
    nz = x > 0
    e[nz] = np.maximum(np.floor(np.log2(x[nz])), -14.0)
    return np.exp2(e - 10.0)


def bound_epi(exact: np.ndarray, alpha: float, abssum: np.ndarray, beta_c: np.ndarray,
              out: str) -> np.ndarray:
    """Acceptance bound of Out = alpha * (A B^T) + beta * C computed with fp32
    sums and an fp32 combine: |alpha| * 1e-4 * abssum for the sum, 2^-22 of
    |alpha * sum| + |beta * C| for the two fp32 roundings of the combine, plus
    one ulp of the output format (bf16 or f16)."""
    b = abs(alpha) * REL_TOL * np.asarray(abssum, np.float64)
    b = b + 2.0 ** -22 * (np.abs(exact) + np.abs(np.asarray(beta_c, np.float64)))
    if out == "bf16":
        b = b + ulp_bf16(exact)
    elif out == "f16":
        b = b + ulp_f16(exact)
    return b


def check_epi(gpu, exact, alpha, abssum, beta_c, out: str):
    """Elementwise acceptance of the epilogue form; (ok, worst err/bound, n bad)."""
    gpu = np.asarray(gpu, np.float64)
    bnd = bound_epi(exact, alpha, abssum, beta_c, out)
    err = np.abs(gpu - np.asarray(exact, np.float64))
    finite = np.isfinite(gpu)
    bad = ~finite | (err > bnd)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bnd > 0, err / bnd, np.where(err > 0, np.inf, 0.0))
    ratio = np.where(finite, ratio, np.inf)
    return int(bad.sum()) == 0, float(ratio.max()) if ratio.size else 0.0, int(bad.sum())


def bound_op(exact: np.ndarray, op: int, alpha: float, abssum: np.ndarray, beta_c: np.ndarray,
             out: str) -> np.ndarray:
    """Acceptance bound of Out = op(alpha * (A B) + beta * C): the fp32 sum and
    combine errors of bound_epi (without its output rounding) carried through
    op with op's largest slope, plus 2^-20 (|x| + |op(x)|) for op evaluated in
    fp32 with the hardware exp / reciprocal and a polynomial erf, plus one
    ulp of a bf16 or fp16 output at op(x).  `exact` is alpha * sum + beta * c."""
    x = np.asarray(exact, np.float64)
    y = apply_op(op, x)
    b = abs(alpha) * REL_TOL * np.asarray(abssum, np.float64)
    b = b + 2.0 ** -22 * (np.abs(x) + np.abs(np.asarray(beta_c, np.float64)))
    b = OP_LIPSCHITZ[int(op)] * b
    if op:
        b = b + 2.0 ** -20 * (np.abs(x) + np.abs(y))
    if out == "bf16":
        b = b + ulp_bf16(y)
    elif out == "f16":
        b = b + ulp_f16(y)
    return b


def check_op(gpu, exact, op, alpha, abssum, beta_c, out: str):
    """Elementwise acceptance of the epilogue with a per-element op;
    (ok, worst err/bound, n bad).  `exact` is the value before op."""
    gpu = np.asarray(gpu, np.float64)
    want = apply_op(op, exact)
    bnd = bound_op(exact, op, alpha, abssum, beta_c, out)
    err = np.abs(gpu - want)
    finite = np.isfinite(gpu)
    bad = ~finite | (err > bnd)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bnd > 0, err / bnd, np.where(err > 0, np.inf, 0.0))
    ratio = np.where(finite, ratio, np.inf)
    return int(bad.sum()) == 0, float(ratio.max()) if ratio.size else 0.0, int(bad.sum())


def bound(ref: np.ndarray, abssum: np.ndarray, out_bf16: bool) -> np.ndarray:
    b = REL_TOL * np.asarray(abssum, np.float64)
    if out_bf16:
        b = b + ulp_bf16(ref)
    return b


def check(gpu: np.ndarray, ref: np.ndarray, abssum: np.ndarray, out_bf16: bool):
    """Elementwise acceptance.  Returns (ok, max(err/bound), n_violations).
    Any NaN or Inf in the GPU output is a violation."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    if gpu.shape != ref.shape:
        raise ValueError(f"shape mismatch {gpu.shape} vs {ref.shape}")
    bnd = bound(ref, abssum, out_bf16)
    err = np.abs(gpu - ref)
    finite = np.isfinite(gpu)
    bad = ~finite | (err > bnd)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bnd > 0, err / bnd, np.where(err > 0, np.inf, 0.0))
    ratio = np.where(finite, ratio, np.inf)
    worst = float(ratio.max()) if ratio.size else 0.0
    nbad = int(bad.sum())
    return nbad == 0, worst, nbad
