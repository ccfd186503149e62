/*
 * tcm.h -- C ABI of libtcm, a tiled dense matrix product Out = A . B^T for
 * AMD Instinct MI355X (gfx950), written in HIP for the CDNA4 matrix cores.
 *
 * The operation is the one the pages state:
 *   - "Blackwell Tensor Cores" (TVM TIRx guide), "The Accumulator's Lifetime":
 *     Out = A @ B.T, float16 inputs, float32 accumulation and output; the
 *     first MMA of a tile ignores the accumulator, so Out is overwritten
 *     (there is no C input and no alpha/beta).
 *   - "API Card: Blackwell Pipeline (tcgen05)" (cuBLASDx), "Descriptor." and
 *     "Host side.": row-major A (M x K), column-major B (K x N, i.e. stored
 *     N x K, "K-major"), row-major C (the TN arrangement); 16-byte alignment
 *     of A, B and C; bfloat16 inputs with float accumulation; batched
 *     problems as in its batched example.
 *   - "Hopper and Blackwell GEMM", Concept "FP8 and FP4, with block scaling"
 *     and its format table: MXFP8 = E4M3 elements with one E8M0 (power of
 *     two) scale per 32 consecutive elements of every row of A and column of
 *     B^T, the scales applied inside the product.
 *
 * Conventions shared by every entry point
 *   Layout     A: M x K row-major (leading dimension K).  B: N x K row-major
 *              (leading dimension K).  Out: M x N row-major (leading dimension
 *              N).  Batched operands are contiguous: problem p starts at
 *              p*M*K, p*N*K and p*M*N elements.  tcm_gemm alone takes other
 *              arrangements and leading dimensions.
 *   Pointers   device pointers (hipMalloc'ed or torch CUDA tensors) on the
 *              current HIP device.  The caller owns all buffers; the library
 *              never allocates, frees or retains them and keeps no per-call
 *              device state.
 *   Alignment  A, B and Out must be 16-byte aligned, and every row of A and
 *              B must be a whole number of 16-byte chunks (K * element size
 *              % 16 == 0); otherwise TCM_ERR_MISALIGNED.  Scale tensors need
 *              no alignment.
 *   Shapes     batch, M, N >= 0 and K >= 0.  A call with batch, M or N equal
 *              to 0 writes nothing and returns TCM_OK.  K == 0 writes zeros.
 *              Sizes whose products overflow, or negative sizes, give
 *              TCM_ERR_INVALID_SHAPE.  K > 2^20 gives TCM_ERR_UNSUPPORTED_SHAPE.
 *              Ragged M and N (not multiples of the tile) are masked.
 *   Execution  every call is asynchronous on `stream` (a hipStream_t; NULL is
 *              the default stream) and does not synchronize.  All arguments
 *              are validated on the host before any HIP call, so invalid
 *              calls return an error without touching the device.  A launch
 *              failure gives TCM_ERR_HIP.  No call falls back silently to
 *              another algorithm: an unsupported request is an error.
 *   Accuracy   element products are exact in fp32; sums are fp32.  The
 *              result r satisfies |r - exact| <= 1e-4 * sum_k |a_ik b_jk| for
 *              fp32 output, plus one bf16 ulp of the exact value for bf16
 *              output (fp32 -> bf16 is round-to-nearest-even).
 *   Threads    thread-safe: the only global state is a per-device cache of
 *              device properties filled once.
 */
#ifndef TCM_H
#define TCM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Result of every call: TCM_OK or the reason the call was refused.  This is
 * the error-or-value form of "API Card: Blackwell Pipeline (tcgen05)", Host
 * side., whose pipeline builder returns either a usable pipeline or an error
 * (one of them that a misaligned operand was given, the card's
 * alignment_unfulfilled, here TCM_ERR_MISALIGNED); unlike the card's
 * Descriptor. gates, a request the fast path cannot take is never served by
 * another algorithm but refused with one of these codes.  Ownership: a plain
 * value; nothing to free. */
typedef enum tcm_status {
    TCM_OK = 0,
    TCM_ERR_NULL_POINTER = 1,      /* a required pointer is NULL */
    TCM_ERR_INVALID_SHAPE = 2,     /* negative size or size products overflow */
    TCM_ERR_UNSUPPORTED_SHAPE = 3, /* valid but not handled (K > 2^20, MX K % 32) */
    TCM_ERR_MISALIGNED = 4,        /* pointer or row length not 16-byte aligned */
    TCM_ERR_UNSUPPORTED_DTYPE = 5, /* dtype / out_dtype pair not supported */
    TCM_ERR_NO_DEVICE = 6,         /* no HIP device, or it is not gfx950 */
    TCM_ERR_HIP = 7,               /* a HIP runtime call or kernel launch failed */
    TCM_ERR_INVALID_ARGUMENT = 8   /* an enumeration argument outside its values */
} tcm_status;

typedef enum tcm_dtype {
    TCM_F16 = 0,  /* IEEE binary16 */
    TCM_BF16 = 1, /* bfloat16 */
    TCM_F32 = 2,  /* IEEE binary32 */
    TCM_E4M3 = 3, /* OCP FP8 E4M3 ("FN": no infinities, max 448) */
    TCM_E8M0 = 4, /* OCP E8M0 scale: 2^(e-127), 0xFF = NaN */
    TCM_E2M1 = 5, /* OCP FP4 E2M1, two per byte, element 2t in the low four bits of
                     byte t (no infinities, no NaN, max 6) */
    TCM_E2M3 = 6, /* OCP FP6 E2M3 (bias 1, 3 mantissa bits, max 7.5), packed: see below */
    TCM_E3M2 = 7  /* OCP FP6 E3M2 (bias 3, 2 mantissa bits, max 28), packed: see below */
} tcm_dtype;

/* Arrangement of a matrix in memory: row-major (the elements of one row
 * contiguous, rows `ld` elements apart) or column-major (columns contiguous,
 * `ld` elements apart). */
typedef enum tcm_order {
    TCM_ROW_MAJOR = 0,
    TCM_COL_MAJOR = 1
} tcm_order;

/* Per-element operation of the epilogue ("API Card: Blackwell Pipeline
 * (tcgen05)", "Device side.": process_and_store(out, op)), applied in fp32 to
 * the finished value x = alpha * sum + beta * c before the rounding to the
 * output type. */
typedef enum tcm_op {
    TCM_OP_IDENTITY = 0,   /* x */
    TCM_OP_RELU = 1,       /* x if x > 0, else 0 */
    TCM_OP_GELU_TANH = 2,  /* x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) */
    TCM_OP_GELU_ERF = 3,   /* x Phi(x), Phi the standard normal distribution function */
    TCM_OP_SILU = 4        /* x / (1 + e^-x) */
} tcm_op;

/*
 * Out = A . B^T for one problem.
 *   A        M x K elements of `dtype` (TCM_F16 or TCM_BF16)
 *   B        N x K elements of `dtype`
 *   Out      M x N elements of `out_dtype` (TCM_F32 or TCM_BF16), overwritten
 * Supported pairs: (F16, F32), (F16, BF16), (BF16, F32), (BF16, BF16).
 */
tcm_status tcm_gemm_tn(const void* A, const void* B, void* Out, int64_t M, int64_t N, int64_t K,
                       tcm_dtype dtype, tcm_dtype out_dtype, void* stream);

/*
 * `batch` independent problems Out[p] = A[p] . B[p]^T, stored contiguously
 * (strides M*K, N*K, M*N elements).  Same dtypes and rules as tcm_gemm_tn;
 * the batched example of "API Card: Blackwell Pipeline (tcgen05)" (intro and
 * Descriptor.: a 128 x 256 x 64 bfloat16 tile, float accumulation, 16-byte
 * alignment) is this call with M = 128, N = 256, K = 64.
 */
tcm_status tcm_batched_gemm_tn(const void* A, const void* B, void* Out, int64_t batch, int64_t M,
                               int64_t N, int64_t K, tcm_dtype dtype, tcm_dtype out_dtype,
                               void* stream);

/*
 * Out = alpha * (A . B^T) + beta * C for one problem: the epilogue with a C
 * input ("API Card: Blackwell Pipeline (tcgen05)", "Device side.": the
 * axpby(alpha, beta, out) accessor; "mma.sync", "Accumulation, transpose and
 * alpha/beta": the scaling after the product, in a stated rounding order).
 *   A, B     as tcm_gemm_tn (dtype TCM_F16 or TCM_BF16)
 *   C        M x N elements of `c_dtype` (TCM_F16, TCM_BF16 or TCM_F32),
 *            16-byte aligned; read only when beta != 0 (then non-NULL)
 *   Out      M x N of `out_dtype` (TCM_F16, TCM_BF16 or TCM_F32), overwritten
 * The product is summed in fp32, combined as alpha * sum + beta * c in fp32,
 * and rounded once to out_dtype (round to nearest even; fp16 overflows to
 * infinity).  C may be Out itself (same pointer and dtype): every element is
 * read before it is written, by the same thread.  Partly overlapping C and
 * Out are not allowed.
 */
tcm_status tcm_gemm_tn_ex(const void* A, const void* B, const void* C, void* Out, int64_t M,
                          int64_t N, int64_t K, tcm_dtype dtype, tcm_dtype c_dtype,
                          tcm_dtype out_dtype, float alpha, float beta, void* stream);

/*
 * General form: Out = op(alpha * (A . B) + beta * C) with A the M x K matrix and B
 * the K x N matrix, each in either arrangement with a leading dimension
 * ("API Card: Blackwell Pipeline (tcgen05)", "Descriptor.": half and bfloat16
 * run in either majorness; "Host side.": global operands are declared
 * row-major or column-major with a leading dimension).
 *   A        element (i, k) at A[i*lda + k] (a_order TCM_ROW_MAJOR, lda >= K)
 *            or A[k*lda + i] (TCM_COL_MAJOR, lda >= M)
 *   B        element (k, j) at B[k*ldb + j] (b_order TCM_ROW_MAJOR, ldb >= N)
 *            or B[j*ldb + k] (TCM_COL_MAJOR, ldb >= K)
 *   C        M x N row-major of `c_dtype`, element (i, j) at C[i*ldc + j],
 *            ldc >= N; read only when beta != 0 (then non-NULL)
 *   Out      M x N row-major of `out_dtype`, element (i, j) at Out[i*ldo + j],
 *            ldo >= N; only these M x N elements are written
 * dtype TCM_F16 or TCM_BF16; c_dtype and out_dtype TCM_F16, TCM_BF16 or
 * TCM_F32.  Sums, combine and rounding as tcm_gemm_tn_ex, with `op` (a tcm_op)
 * applied in fp32 between the combine and the rounding: ReLU exactly, the
 * others from the hardware exponential and reciprocal (and, for
 * TCM_OP_GELU_ERF, the erfc approximation of Abramowitz and Stegun 7.1.26,
 * absolute error <= 1.5e-7), within 2^-20 (|x| + |op(x)|).  C may be Out itself
 * (same pointer, dtype and leading dimension).  Row-major A with
 * column-major B (lda = ldb = K, ldo = N) is tcm_gemm_tn's operation.
 * Every leading dimension must be at least 1 and at least the size named
 * above (TCM_ERR_INVALID_SHAPE), lda and ldb at most 2^21 and ldo and ldc
 * below 2^31 (TCM_ERR_UNSUPPORTED_SHAPE); an order or op outside its values
 * gives TCM_ERR_INVALID_ARGUMENT.  Alignment: A, B, Out (and C when read) 16-byte
 * aligned, lda and ldb multiples of 8 elements, and K a multiple of 8 unless
 * A is column-major and B row-major (TCM_ERR_MISALIGNED); ldo and ldc are
 * free.
 */
tcm_status tcm_gemm(const void* A, tcm_order a_order, int64_t lda, const void* B,
                    tcm_order b_order, int64_t ldb, const void* C, int64_t ldc, void* Out,
                    int64_t ldo, int64_t M, int64_t N, int64_t K, tcm_dtype dtype,
                    tcm_dtype c_dtype, tcm_dtype out_dtype, float alpha, float beta, tcm_op op,
                    void* stream);

/*
 * MXFP8 block-scaled Out = (A * SA) . (B * SB)^T.
 *   A        M x K E4M3 bytes;  B  N x K E4M3 bytes
 *   scale_A  M x (K/32) E8M0 bytes, row-major: scale_A[i][q] multiplies
 *            A[i][32q .. 32q+31]
 *   scale_B  N x (K/32) E8M0 bytes: scale_B[j][q] multiplies B[j][32q .. 32q+31]
 *   Out      M x N of `out_dtype` (TCM_F32 or TCM_BF16)
 * K must be a multiple of 32 (TCM_ERR_UNSUPPORTED_SHAPE otherwise).  A NaN
 * scale (0xFF) or element makes the affected outputs NaN.
 */
tcm_status tcm_gemm_mx_fp8(const void* A, const void* B, const void* scale_A, const void* scale_B,
                           void* Out, int64_t M, int64_t N, int64_t K, tcm_dtype out_dtype,
                           void* stream);

/*
 * MXFP4 block-scaled Out = (A * SA) . (B * SB)^T ("Hopper and Blackwell GEMM",
 * Concept, "FP8 and FP4, with block scaling": the MXFP4 row of its format
 * table, E2M1 elements with one E8M0 scale per 32).
 *   A        M x K E2M1 elements stored M x (K/2) bytes (TCM_E2M1 packing)
 *   B        N x K E2M1 elements stored N x (K/2) bytes
 *   scale_A, scale_B, Out, K, errors: as tcm_gemm_mx_fp8.
 */
tcm_status tcm_gemm_mx_fp4(const void* A, const void* B, const void* scale_A, const void* scale_B,
                           void* Out, int64_t M, int64_t N, int64_t K, tcm_dtype out_dtype,
                           void* stream);

/*
 * MXFP6 block-scaled Out = (A * SA) . (B * SB)^T (the 6-bit element formats of
 * the scaled MMA kind mxf8f6f4 named in "Hopper and Blackwell GEMM", Concept,
 * "FP8 and FP4, with block scaling"; OCP FP6 with one E8M0 scale per 32).
 *   elem_dtype  TCM_E2M3 or TCM_E3M2, for both A and B
 *   A        M x K codes packed as one little-endian bit stream per row: element
 *            t of a row in bits 6t .. 6t+5 of its bytes (four elements per
 *            three bytes), M x (3K/4) bytes
 *   B        N x K codes packed the same way, N x (3K/4) bytes
 *   scale_A, scale_B, Out, errors: as tcm_gemm_mx_fp8, except that K must be a
 *            multiple of 64 (rows of whole 16-byte pieces; TCM_ERR_MISALIGNED
 *            when K % 32 == 0 but K % 64 != 0).
 */
tcm_status tcm_gemm_mx_fp6(const void* A, const void* B, const void* scale_A, const void* scale_B,
                           void* Out, int64_t M, int64_t N, int64_t K, tcm_dtype elem_dtype,
                           tcm_dtype out_dtype, void* stream);

/*
 * MXFP8 with operands in either arrangement and leading dimensions:
 * Out = (A * SA) . (B * SB) with A the M x K and B the K x N matrix of E4M3
 * elements ("API Card: Blackwell Pipeline (tcgen05)", Descriptor.: fp8
 * types, like the 16-bit ones, reach the fast path in either majorness;
 * "Hopper and Blackwell GEMM", Concept, FP8 and FP4 with block scaling).
 *   A        a_order TCM_ROW_MAJOR: A[i * lda + k] (K contiguous, lda >= K);
 *            TCM_COL_MAJOR: A[k * lda + i] (M contiguous, lda >= M)
 *   B        b_order TCM_ROW_MAJOR: B[k * ldb + j] (N contiguous, ldb >= N);
 *            TCM_COL_MAJOR: B[j * ldb + k] (K contiguous, ldb >= K: the TN
 *            form of tcm_gemm_mx_fp8)
 *   scale_A  M x (K/32) E8M0 bytes: scale_A[i][q] multiplies a(i, 32q .. 32q+31)
 *   scale_B  N x (K/32) E8M0 bytes: scale_B[j][q] multiplies b(32q .. 32q+31, j)
 *            (the scale layout does not depend on the arrangement)
 *   Out      M x N of out_dtype (TCM_F32 or TCM_BF16), row-major, rows ldo >= N
 *            apart, overwritten
 * elem_dtype must be TCM_E4M3 (TCM_ERR_UNSUPPORTED_DTYPE otherwise).  K must
 * be a multiple of 32 (TCM_ERR_UNSUPPORTED_SHAPE); lda and ldb are multiples
 * of 16 and A, B, Out 16-byte aligned (TCM_ERR_MISALIGNED); lda, ldb <= 2^21
 * (TCM_ERR_UNSUPPORTED_SHAPE); a leading dimension below its minimum is
 * TCM_ERR_INVALID_SHAPE and an unknown order TCM_ERR_INVALID_ARGUMENT.  Sums
 * and rounding as tcm_gemm_mx_fp8, which dense TN storage (A row-major with
 * lda = K, B column-major with ldb = K, ldo = N) runs exactly.
 */
tcm_status tcm_gemm_mx(const void* A, tcm_order a_order, int64_t lda, const void* B,
                       tcm_order b_order, int64_t ldb, const void* scale_A, const void* scale_B,
                       void* Out, int64_t ldo, int64_t M, int64_t N, int64_t K,
                       tcm_dtype elem_dtype, tcm_dtype out_dtype, void* stream);

/*
 * NVFP4 Out = gA gB (A * SA) . (B * SB)^T ("Hopper and Blackwell GEMM",
 * Concept, "FP8 and FP4, with block scaling": the format table's NVFP4 row,
 * E2M1 elements with an E4M3 scale per 16 values and one FP32 scale per
 * tensor).
 *   A        M x K E2M1 elements stored M x (K/2) bytes (TCM_E2M1 packing)
 *   B        N x K E2M1 elements stored N x (K/2) bytes
 *   scale_A  M x (K/16) E4M3 bytes: scale_A[i][q] multiplies A[i][16q .. 16q+15]
 *   scale_B  N x (K/16) E4M3 bytes; both 2-byte aligned
 *   global_scale_A, global_scale_B  the per-tensor scales gA, gB
 *   Out      M x N of `out_dtype` (TCM_F16, TCM_BF16 or TCM_F32), overwritten
 * K must be a multiple of 32 (TCM_ERR_UNSUPPORTED_SHAPE).  Each element times
 * its block scale is exact in fp16; the products are summed in fp32 and
 * multiplied by the fp32 product gA gB before the one rounding to out_dtype.
 * With K a multiple of 256 and both scale tensors 16-byte aligned, a faster
 * form reads each row's scales of 256 K values at once; where such a product
 * also has enough 256 x 256 tiles to fill the device, a kernel that keeps the
 * elements 4-bit in LDS and converts them per fragment runs instead (its
 * fp32 sums run in another order, within the same bound).
 */
tcm_status tcm_gemm_nvfp4(const void* A, const void* B, const void* scale_A, const void* scale_B,
                          float global_scale_A, float global_scale_B, void* Out, int64_t M,
                          int64_t N, int64_t K, tcm_dtype out_dtype, void* stream);

/* What a call with these arguments would launch (host only: no HIP call when
 * num_cus > 0; num_cus == 0 asks the current device for its CU count). */
typedef struct tcm_plan {
    int32_t tile_m, tile_n, tile_k; /* output tile and K slice per stage */
    int32_t stages;                 /* depth of the LDS operand ring */
    int32_t threads;                /* threads per workgroup */
    int32_t stage_bytes;            /* LDS bytes of one stage (A tile + B tile) */
    int32_t lds_bytes;              /* LDS bytes of the operand ring (stages x stage_bytes);
                                       output staging and MX scale buffers add to it, within
                                       the 160 KiB of a compute unit */
    int32_t grid;                   /* workgroups launched (persistent when < tiles) */
    int64_t tiles;                  /* output tiles over all problems */
    int32_t kernel;                 /* internal kernel variant id */
} tcm_plan;

/* mx == 1 plans tcm_gemm_mx_fp8 and mx == 2 tcm_gemm_mx_fp4 (with 16-byte aligned
 * scale tensors), mx == 3 tcm_gemm_mx_fp6 (with 16-byte aligned scale tensors where
 * K % 512 == 0, else 4-byte aligned), mx == 4 tcm_gemm_nvfp4 (with 16-byte aligned scale
 * tensors), mx == 5 tcm_gemm_mx with an M- or N-major operand (dtype is then ignored);
 * other mx values are TCM_ERR_INVALID_ARGUMENT. */
tcm_status tcm_plan_gemm(int64_t batch, int64_t M, int64_t N, int64_t K, tcm_dtype dtype,
                         tcm_dtype out_dtype, int mx, int num_cus, tcm_plan* plan);

/* Static, human-readable name of a status code, the counterpart of the error
 * string lookup of "API Card: Blackwell Pipeline (tcgen05)", Host side.
 * (which names the card's error values, alignment_unfulfilled among them).
 * Codes outside the enumeration give "TCM_ERR_UNKNOWN: unknown status code".  The string is
 * static and owned by the library (never NULL, never freed by the caller);
 * the call touches no device and is thread-safe. */
const char* tcm_status_string(tcm_status s);

#ifdef __cplusplus
}
#endif

#endif /* TCM_H */
