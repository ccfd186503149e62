/*
 * oracle.c -- plain, slow fp64 CPU reference for the tiled matrix product
 * Out = A . B^T.  TEST INFRASTRUCTURE ONLY: nothing in the product library
 * links, includes or calls this file; only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark do.  It shares no code, header, table or
 * helper with the HIP path.
 *
 * What it computes (the plain definition, no blocking, no reordering):
 *
 *   ref[i][j]    = sum_{k=0}^{K-1} a(i,k) * b(j,k)      fp64, k ascending
 *   abssum[i][j] = sum_{k=0}^{K-1} |a(i,k) * b(j,k)|    fp64, for tolerances
 *
 * where a(i,k), b(j,k) are the exact real values of the stored input
 * elements.  B is stored N x K ("K-major"): the product uses B transposed.
 *   - "Blackwell Tensor Cores" (TVM TIRx guide), "The Accumulator's
 *     Lifetime": the example computes Out = A @ B.T with A (128, 64) and
 *     B (64, 64), float16 in, float32 out; the first MMA ignores the previous
 *     accumulator contents, so there is no C input.
 *   - "mma.sync" (TVM TIRx tile-op reference), "Operand coordinates and
 *     ownership": B's logical axes are (N, K) although the product uses B
 *     transposed.
 *   - "API Card: Blackwell Pipeline (tcgen05)" (cuBLASDx), "Descriptor.":
 *     row-major A, column-major B (K x N), i.e. the TN arrangement.
 *
 * Block-scaled (MX) inputs follow "Hopper and Blackwell GEMM", Concept
 * section "FP8 and FP4, with block scaling" and its format table: every row
 * of A and column of B (= row of the N x K storage) is cut into blocks of 32
 * consecutive K elements and each block's values are multiplied by their own
 * E8M0 scale, a power of two:
 *
 *   a(i,k) = e4m3(A[i][k]) * e8m0(SA[i][k/32])
 *   b(j,k) = e4m3(B[j][k]) * e8m0(SB[j][k/32])
 *
 * and the same with E2M1 (MXFP4, the format table's 4-bit row) or the FP6
 * formats E2M3 and E3M2 (MXFP6, the 6-bit rows) in place of E4M3.
 *
 * Element decoders are written from the format definitions (IEEE 754
 * binary16; bfloat16 = the upper half of binary32; OCP MX E4M3 "FN" with bias
 * 7, no infinities, S.1111.111 = NaN; OCP MX E2M1 with bias 1, no infinities
 * or NaN; E8M0 = 2^(e-127), 0xFF = NaN).  The page table names these formats
 * but does not print their bit layouts; the OCP Microscaling specification
 * cited in that page's "Go deeper" list does.  E2M1 elements are stored two
 * per byte, element 2t in the low four bits of byte t and element 2t + 1 in
 * the high four bits (the pages fix no packing; this is the plainest
 * little-endian reading), so a row of K elements is K/2 bytes.  FP6 codes
 * (E2M3: bias 1, 3 mantissa bits, max 7.5; E3M2: bias 3, 2 mantissa bits,
 * max 28; neither has infinities or NaN) are stored as one little-endian bit
 * stream, element t in bits 6t .. 6t+5, so a row of K elements is 3K/4 bytes
 * and a 32-element block 24 bytes.
 *
 * Accuracy: sequential fp64 summation errs by at most about K * 2^-53 *
 * abssum, far below any tolerance used against the GPU path.  Every MX
 * product is exact in fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F16 = 0, OR_BF16 = 1, OR_F32 = 2, OR_E4M3 = 3, OR_E8M0 = 4, OR_E2M1 = 5, OR_E2M3 = 6,
       OR_E3M2 = 7 };

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
static double dec_f16(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m/1024 * 2^-14 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return s ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa bits. */
static double dec_bf16(uint16_t h) {
    int s = h >> 15, e = (h >> 7) & 0xff, m = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133); /* m/128 * 2^-126 */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134); /* (1 + m/128) * 2^(e-127) */
    return s ? -v : v;
}

/* OCP E4M3 (FN): 1 sign, 4 exponent (bias 7), 3 mantissa; no infinities;
 * exponent 1111 with mantissa 111 is NaN; max normal 448. */
static double dec_e4m3(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 0xf, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9); /* m/8 * 2^-6 */
    else
        v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* OCP E8M0: unsigned exponent only, 2^(e-127); 0xFF is NaN. */
/* OCP E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent field 0
 * holds the subnormal 0.5 * m; no infinities, no NaN. */
static double dec_e2m1(unsigned nib) {
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* OCP FP6 E2M3: 1 sign, 2 exponent (bias 1), 3 mantissa bits; exponent
 * field 0 holds the subnormals m/8; no infinities, no NaN; max 7.5. */
static double dec_e2m3(unsigned c) {
    int s = (c >> 5) & 1, e = (c >> 3) & 3, m = c & 7;
    double v = e == 0 ? m / 8.0 : ldexp(1.0 + m / 8.0, e - 1);
    return s ? -v : v;
}

/* OCP FP6 E3M2: 1 sign, 3 exponent (bias 3), 2 mantissa bits; exponent
 * field 0 holds the subnormals m/4 * 2^-2; no infinities, no NaN; max 28. */
static double dec_e3m2(unsigned c) {
    int s = (c >> 5) & 1, e = (c >> 2) & 7, m = c & 3;
    double v = e == 0 ? ldexp(m / 4.0, -2) : ldexp(1.0 + m / 4.0, e - 3);
    return s ? -v : v;
}

/* 6-bit code `idx` of a packed FP6 array: bits 6 idx .. 6 idx + 5 of the
 * byte string read as one little-endian bit stream (element 4t in the low six
 * bits of byte 3t; four elements per three bytes). */
static unsigned fp6_code(const uint8_t* b, int64_t idx) {
    const int64_t bit = 6 * idx;
    const unsigned lo = b[bit / 8];
    const unsigned hi = (bit % 8) > 2 ? b[bit / 8 + 1] : 0;
    return ((lo | (hi << 8)) >> (bit % 8)) & 0x3f;
}

static double dec_e8m0(uint8_t b) {
    if (b == 0xff)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

static double dec_f32(uint32_t w) {
    float f;
    memcpy(&f, &w, 4);
    return (double)f;
}

/* Storage bits per element. */
static int elem_bits(int dtype) {
    switch (dtype) {
    case OR_F16:
    case OR_BF16:
        return 16;
    case OR_F32:
        return 32;
    case OR_E4M3:
    case OR_E8M0:
        return 8;
    case OR_E2M1:
        return 4;
    case OR_E2M3:
    case OR_E3M2:
        return 6;
    }
    return 0;
}

static double dec_one(int dtype, const void* src, int64_t idx) {
    switch (dtype) {
    case OR_F16:
        return dec_f16(((const uint16_t*)src)[idx]);
    case OR_BF16:
        return dec_bf16(((const uint16_t*)src)[idx]);
    case OR_F32:
        return dec_f32(((const uint32_t*)src)[idx]);
    case OR_E4M3:
        return dec_e4m3(((const uint8_t*)src)[idx]);
    case OR_E8M0:
        return dec_e8m0(((const uint8_t*)src)[idx]);
    case OR_E2M1: {
        uint8_t byte = ((const uint8_t*)src)[idx / 2];
        return dec_e2m1((idx & 1) ? byte >> 4 : byte & 0xF);
    }
    case OR_E2M3:
        return dec_e2m3(fp6_code((const uint8_t*)src, idx));
    case OR_E3M2:
        return dec_e3m2(fp6_code((const uint8_t*)src, idx));
    }
    return NAN;
}

/* Decode n stored elements of the given format into exact fp64 values. */
int oracle_decode(int dtype, const void* src, int64_t n, double* dst) {
    if (!elem_bits(dtype) || (n > 0 && (!src || !dst)))
        return -1;
    for (int64_t i = 0; i < n; ++i)
        dst[i] = dec_one(dtype, src, i);
    return 0;
}

/* Exact real value of operand element (r, k) of an R x K matrix: the element
 * itself, times its block's E8M0 scale when a scale tensor is given. */
static double operand_value(int dtype, const void* X, const uint8_t* SX, int64_t K, int64_t r,
                            int64_t k) {
    double v = dec_one(dtype, X, r * K + k);
    if (SX)
        v *= dec_e8m0(SX[r * (K / 32) + k / 32]);
    return v;
}

/* Decode rows [r0, r1) of an R x K operand into dst (row-major). */
static void decode_rows(int dtype, const void* X, const uint8_t* SX, int64_t K, int64_t r0,
                        int64_t r1, double* dst) {
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t k = 0; k < K; ++k)
            dst[(r - r0) * K + k] = operand_value(dtype, X, SX, K, r, k);
}

typedef struct {
    const double *a, *b; /* decoded A (M x K) and B (N x K) */
    int64_t M, N, K;
    double *ref, *abssum;
    int64_t row0, row1;
} job_t;

/* The definition itself: for each (i, j), a sequential fp64 sum over k. */
static void* rows_worker(void* p) {
    job_t* j = (job_t*)p;
    for (int64_t i = j->row0; i < j->row1; ++i) {
        const double* ai = j->a + i * j->K;
        for (int64_t c = 0; c < j->N; ++c) {
            const double* bc = j->b + c * j->K;
            double s = 0.0, sa = 0.0;
            for (int64_t k = 0; k < j->K; ++k) {
                double prod = ai[k] * bc[k];
                s += prod;
                sa += fabs(prod);
            }
            if (j->ref)
                j->ref[i * j->N + c] = s;
            if (j->abssum)
                j->abssum[i * j->N + c] = sa;
        }
    }
    return NULL;
}

static int run_rows(const double* a, const double* b, int64_t M, int64_t N, int64_t K, double* ref,
                    double* abssum, int nthreads) {
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > M)
        nthreads = (int)(M > 0 ? M : 1);
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
    if (!th || !jobs) {
        free(th);
        free(jobs);
        return -2;
    }
    int started = 0, rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (job_t){a, b, M, N, K, ref, abssum, M * t / nthreads, M * (t + 1) / nthreads};
        if (pthread_create(&th[t], NULL, rows_worker, &jobs[t]) != 0) {
            rc = -3;
            break;
        }
        ++started;
    }
    for (int t = 0; t < started; ++t)
        pthread_join(th[t], NULL);
    free(th);
    free(jobs);
    return rc;
}

/* One problem: decode both operands exactly, then apply the definition. */
static int gemm_one(int dtype, const void* A, const void* B, const uint8_t* SA, const uint8_t* SB,
                    int64_t M, int64_t N, int64_t K, double* ref, double* abssum, int nthreads) {
    double* a = (double*)malloc((size_t)(M * K > 0 ? M * K : 1) * sizeof(double));
    double* b = (double*)malloc((size_t)(N * K > 0 ? N * K : 1) * sizeof(double));
    if (!a || !b) {
        free(a);
        free(b);
        return -2;
    }
    decode_rows(dtype, A, SA, K, 0, M, a);
    decode_rows(dtype, B, SB, K, 0, N, b);
    int rc = run_rows(a, b, M, N, K, ref, abssum, nthreads);
    free(a);
    free(b);
    return rc;
}

static int shape_ok(int64_t batch, int64_t M, int64_t N, int64_t K) {
    return batch >= 1 && M >= 1 && N >= 1 && K >= 0;
}

/*
 * Batched plain GEMM: batch independent problems stored contiguously
 * (strides M*K, N*K and M*N elements).  dtype is OR_F16, OR_BF16 or OR_F32.
 * ref / abssum (either may be NULL) receive batch*M*N fp64 values.
 */
int oracle_gemm_tn(int dtype, const void* A, const void* B, int64_t batch, int64_t M, int64_t N,
                   int64_t K, double* ref, double* abssum, int nthreads) {
    if (!(dtype == OR_F16 || dtype == OR_BF16 || dtype == OR_F32) || !A || !B ||
        !shape_ok(batch, M, N, K))
        return -1;
    int es = elem_bits(dtype) / 8;
    for (int64_t p = 0; p < batch; ++p) {
        int rc = gemm_one(dtype, (const char*)A + p * M * K * es, (const char*)B + p * N * K * es,
                          NULL, NULL, M, N, K, ref ? ref + p * M * N : NULL,
                          abssum ? abssum + p * M * N : NULL, nthreads);
        if (rc)
            return rc;
    }
    return 0;
}

/* MX block-scaled GEMM with elements of format `dtype` (OR_E4M3, OR_E2M1,
 * OR_E2M3 or OR_E3M2),
 * one E8M0 scale per 32 consecutive K elements of every row of A
 * (SA: M x K/32) and of B (SB: N x K/32). */
int oracle_gemm_mx_typed(int dtype, const uint8_t* A, const uint8_t* B, const uint8_t* SA,
                         const uint8_t* SB, int64_t M, int64_t N, int64_t K, double* ref,
                         double* abssum, int nthreads) {
    if (!(dtype == OR_E4M3 || dtype == OR_E2M1 || dtype == OR_E2M3 || dtype == OR_E3M2) || !A ||
        !B || !SA || !SB ||
        !shape_ok(1, M, N, K) || K % 32 != 0)
        return -1;
    return gemm_one(dtype, A, B, SA, SB, M, N, K, ref, abssum, nthreads);
}

/* The E4M3 form. */
int oracle_gemm_mx(const uint8_t* A, const uint8_t* B, const uint8_t* SA, const uint8_t* SB,
                   int64_t M, int64_t N, int64_t K, double* ref, double* abssum, int nthreads) {
    return oracle_gemm_mx_typed(OR_E4M3, A, B, SA, SB, M, N, K, ref, abssum, nthreads);
}

/*
 * Epilogue with a C input.  "API Card: Blackwell Pipeline (tcgen05)",
 * "Device side.", lists an axpby(alpha, beta, out) accessor among the
 * epilogue's operations, and "mma.sync", "Accumulation, transpose and
 * alpha/beta", places alpha/beta scaling after the product at the call site.
 * Read plainly (the BLAS axpby), with C the output's prior contents:
 *
 *   out[t] = alpha * ref[t] + beta * c(t)       fp64, exact up to one rounding
 *
 * where c(t) is the exact value of stored element t of C (format c_dtype,
 * OR_F16, OR_BF16 or OR_F32).  C may be NULL when beta == 0.
 */
int oracle_axpby(int64_t n, double alpha, const double* ref, double beta, int c_dtype,
                 const void* C, double* out) {
    if (n < 0 || (n > 0 && (!ref || !out)) ||
        (beta != 0.0 && (!C || !(c_dtype == OR_F16 || c_dtype == OR_BF16 || c_dtype == OR_F32))))
        return -1;
    for (int64_t t = 0; t < n; ++t) {
        double v = alpha * ref[t];
        if (beta != 0.0)
            v += beta * dec_one(c_dtype, C, t);
        out[t] = v;
    }
    return 0;
}

/*
 * Selected entries only, for problems too large to compute whole: entry t is
 * (row ii[t], column jj[t]) of problem bb[t] (bb may be NULL for batch 1).
 * SA/SB non-NULL selects the MX definition (dtype must then be OR_E4M3 or
 * OR_E2M1, OR_E2M3, OR_E3M2).
 */
int oracle_entries(int dtype, const void* A, const void* B, const uint8_t* SA, const uint8_t* SB,
                   int64_t M, int64_t N, int64_t K, const int64_t* bb, const int64_t* ii,
                   const int64_t* jj, int64_t n, double* ref, double* abssum) {
    if (!elem_bits(dtype) || !A || !B || !ii || !jj || !shape_ok(1, M, N, K) ||
        ((SA || SB) &&
         (!SA || !SB ||
          !(dtype == OR_E4M3 || dtype == OR_E2M1 || dtype == OR_E2M3 || dtype == OR_E3M2) ||
          K % 32 != 0)) ||
        ((dtype == OR_E2M1 || dtype == OR_E2M3 || dtype == OR_E3M2) && (!SA || K % 4 != 0)))
        return -1;
    const int64_t bits = elem_bits(dtype);
    for (int64_t t = 0; t < n; ++t) {
        int64_t p = bb ? bb[t] : 0, i = ii[t], j = jj[t];
        if (p < 0 || i < 0 || i >= M || j < 0 || j >= N || (SA && p != 0))
            return -1;
        const char* Ap = (const char*)A + p * M * K * bits / 8;
        const char* Bp = (const char*)B + p * N * K * bits / 8;
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double prod = operand_value(dtype, Ap, SA, K, i, k) * operand_value(dtype, Bp, SB, K, j, k);
            s += prod;
            sa += fabs(prod);
        }
        if (ref)
            ref[t] = s;
        if (abssum)
            abssum[t] = sa;
    }
    return 0;
}

/*
 * Operands in either arrangement, with leading dimensions.  "API Card:
 * Blackwell Pipeline (tcgen05)", "Descriptor." and "Host side.": the product
 * is Out = A . B with A the M x K matrix and B the K x N matrix; each global
 * operand is declared row-major or column-major and takes a leading dimension
 * (the elements from one stored row, or column, to the next), and the 16-bit
 * types run in either arrangement.  Read plainly, as in BLAS:
 *
 *   a(i,k) = A[i * lda + k]   row-major A      A[k * lda + i]   column-major A
 *   b(k,j) = B[k * ldb + j]   row-major B      B[j * ldb + k]   column-major B
 *
 *   ref[i][j] = sum_k a(i,k) * b(k,j),   abssum likewise, fp64, k ascending
 *
 * The TN arrangement of oracle_gemm_tn is row-major A with lda = K and
 * column-major B with ldb = K.  A row-major matrix needs ld >= its column
 * count, a column-major one ld >= its row count.
 */
enum { OR_ROW_MAJOR = 0, OR_COL_MAJOR = 1 };

static int64_t a_index(int order, int64_t ld, int64_t i, int64_t k) {
    return order == OR_ROW_MAJOR ? i * ld + k : k * ld + i;
}

static int64_t b_index(int order, int64_t ld, int64_t k, int64_t j) {
    return order == OR_ROW_MAJOR ? k * ld + j : j * ld + k;
}

static int ld_ok(int dtype, int a_order, int64_t lda, int b_order, int64_t ldb, int64_t M,
                 int64_t N, int64_t K) {
    if (!(dtype == OR_F16 || dtype == OR_BF16 || dtype == OR_F32) || !shape_ok(1, M, N, K))
        return 0;
    if ((a_order != OR_ROW_MAJOR && a_order != OR_COL_MAJOR) ||
        (b_order != OR_ROW_MAJOR && b_order != OR_COL_MAJOR))
        return 0;
    return lda >= (a_order == OR_ROW_MAJOR ? K : M) && lda >= 1 &&
           ldb >= (b_order == OR_ROW_MAJOR ? N : K) && ldb >= 1;
}

int oracle_gemm_ld(int dtype, const void* A, int a_order, int64_t lda, const void* B, int b_order,
                   int64_t ldb, int64_t M, int64_t N, int64_t K, double* ref, double* abssum,
                   int nthreads) {
    if (!A || !B || !ld_ok(dtype, a_order, lda, b_order, ldb, M, N, K))
        return -1;
    /* gather the logical matrices: a as M x K, b as N x K (b's row j holds
     * column j of B), then the same sums as the TN form */
    double* a = (double*)malloc((size_t)(M * K > 0 ? M * K : 1) * sizeof(double));
    double* b = (double*)malloc((size_t)(N * K > 0 ? N * K : 1) * sizeof(double));
    if (!a || !b) {
        free(a);
        free(b);
        return -2;
    }
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k)
            a[i * K + k] = dec_one(dtype, A, a_index(a_order, lda, i, k));
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k)
            b[j * K + k] = dec_one(dtype, B, b_index(b_order, ldb, k, j));
    int rc = run_rows(a, b, M, N, K, ref, abssum, nthreads);
    free(a);
    free(b);
    return rc;
}

/* Selected entries (ii[t], jj[t]) of the same product, one by one. */
int oracle_entries_ld(int dtype, const void* A, int a_order, int64_t lda, const void* B,
                      int b_order, int64_t ldb, int64_t M, int64_t N, int64_t K, const int64_t* ii,
                      const int64_t* jj, int64_t n, double* ref, double* abssum) {
    if (!A || !B || !ii || !jj || !ld_ok(dtype, a_order, lda, b_order, ldb, M, N, K))
        return -1;
    for (int64_t t = 0; t < n; ++t) {
        int64_t i = ii[t], j = jj[t];
        if (i < 0 || i >= M || j < 0 || j >= N)
            return -1;
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double prod = dec_one(dtype, A, a_index(a_order, lda, i, k)) *
                          dec_one(dtype, B, b_index(b_order, ldb, k, j));
            s += prod;
            sa += fabs(prod);
        }
        if (ref)
            ref[t] = s;
        if (abssum)
            abssum[t] = sa;
    }
    return 0;
}

/*
 * MXFP8 operands in either arrangement.  "API Card: Blackwell Pipeline
 * (tcgen05)", "Descriptor.": fp8 types, like the 16-bit ones, reach the fast
 * path in either majorness; "Hopper and Blackwell GEMM", Concept, "FP8 and
 * FP4, with block scaling": the scale blocks run along K, one per 32
 * elements of a row of A and of a column of B, whatever the elements'
 * storage.  So, with the element index of the arrangement above:
 *
 *   a(i,k) = e4m3(A[a_index]) * e8m0(SA[i * (K/32) + k/32])
 *   b(k,j) = e4m3(B[b_index]) * e8m0(SB[j * (K/32) + k/32])
 *
 * (SA is M x K/32 and SB N x K/32 in both arrangements), then the same sums.
 */
static int mx_ld_ok(int a_order, int64_t lda, int b_order, int64_t ldb, int64_t M, int64_t N,
                    int64_t K) {
    if (!shape_ok(1, M, N, K) || K % 32 != 0)
        return 0;
    if ((a_order != OR_ROW_MAJOR && a_order != OR_COL_MAJOR) ||
        (b_order != OR_ROW_MAJOR && b_order != OR_COL_MAJOR))
        return 0;
    return lda >= (a_order == OR_ROW_MAJOR ? K : M) && lda >= 1 &&
           ldb >= (b_order == OR_ROW_MAJOR ? N : K) && ldb >= 1;
}

static double mx_a(const uint8_t* A, int a_order, int64_t lda, const uint8_t* SA, int64_t K,
                   int64_t i, int64_t k) {
    return dec_e4m3(A[a_index(a_order, lda, i, k)]) * dec_e8m0(SA[i * (K / 32) + k / 32]);
}

static double mx_b(const uint8_t* B, int b_order, int64_t ldb, const uint8_t* SB, int64_t K,
                   int64_t k, int64_t j) {
    return dec_e4m3(B[b_index(b_order, ldb, k, j)]) * dec_e8m0(SB[j * (K / 32) + k / 32]);
}

int oracle_gemm_mx_ld(const uint8_t* A, int a_order, int64_t lda, const uint8_t* B, int b_order,
                      int64_t ldb, const uint8_t* SA, const uint8_t* SB, int64_t M, int64_t N,
                      int64_t K, double* ref, double* abssum, int nthreads) {
    if (!A || !B || !SA || !SB || !mx_ld_ok(a_order, lda, b_order, ldb, M, N, K))
        return -1;
    double* a = (double*)malloc((size_t)(M * K > 0 ? M * K : 1) * sizeof(double));
    double* b = (double*)malloc((size_t)(N * K > 0 ? N * K : 1) * sizeof(double));
    if (!a || !b) {
        free(a);
        free(b);
        return -2;
    }
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k)
            a[i * K + k] = mx_a(A, a_order, lda, SA, K, i, k);
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k)
            b[j * K + k] = mx_b(B, b_order, ldb, SB, K, k, j);
    int rc = run_rows(a, b, M, N, K, ref, abssum, nthreads);
    free(a);
    free(b);
    return rc;
}

int oracle_entries_mx_ld(const uint8_t* A, int a_order, int64_t lda, const uint8_t* B,
                         int b_order, int64_t ldb, const uint8_t* SA, const uint8_t* SB,
                         int64_t M, int64_t N, int64_t K, const int64_t* ii, const int64_t* jj,
                         int64_t n, double* ref, double* abssum) {
    if (!A || !B || !SA || !SB || !ii || !jj || !mx_ld_ok(a_order, lda, b_order, ldb, M, N, K))
        return -1;
    for (int64_t t = 0; t < n; ++t) {
        int64_t i = ii[t], j = jj[t];
        if (i < 0 || i >= M || j < 0 || j >= N)
            return -1;
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double prod = mx_a(A, a_order, lda, SA, K, i, k) * mx_b(B, b_order, ldb, SB, K, k, j);
            s += prod;
            sa += fabs(prod);
        }
        if (ref)
            ref[t] = s;
        if (abssum)
            abssum[t] = sa;
    }
    return 0;
}

/*
 * Per-element operation of the epilogue.  "API Card: Blackwell Pipeline
 * (tcgen05)", "Device side.", lists process_and_store(out, op) among the
 * epilogue accessors: an operation applied to every result element as it is
 * stored.  The pages name no particular operation; this oracle defines the
 * usual activation functions from their mathematical definitions, applied to
 * the finished value alpha * sum + beta * c:
 *
 *   0 identity   x
 *   1 relu       x if x > 0, else 0
 *   2 gelu_tanh  x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3)))
 *                (the tanh form of the Gaussian error linear unit,
 *                Hendrycks and Gimpel)
 *   3 gelu_erf   x * Phi(x) = x/2 * erfc(-x / sqrt(2))   (Phi the standard
 *                normal distribution function; erfc avoids cancelling
 *                1 + erf for negative x)
 *   4 silu       x / (1 + exp(-x))
 *
 * fp64 with the C library's tanh, erfc and exp.
 */
int oracle_apply_op(int64_t n, int op, const double* x, double* out) {
    if (n < 0 || (n > 0 && (!x || !out)) || op < 0 || op > 4)
        return -1;
    const double k_tanh = sqrt(2.0 / (4.0 * atan(1.0)));  /* sqrt(2 / pi) */
    for (int64_t t = 0; t < n; ++t) {
        const double v = x[t];
        double y;
        switch (op) {
        case 1: y = v > 0.0 ? v : 0.0; break;
        case 2: y = 0.5 * v * (1.0 + tanh(k_tanh * (v + 0.044715 * v * v * v))); break;
        case 3: y = 0.5 * v * erfc(-v / sqrt(2.0)); break;
        case 4: y = v / (1.0 + exp(-v)); break;
        default: y = v;
        }
        out[t] = y;
    }
    return 0;
}

/*
 * NVFP4 ("Hopper and Blackwell GEMM", Concept, "FP8 and FP4, with block
 * scaling", the format table's NVFP4 row): E2M1 elements (stored as for
 * MXFP4, two per byte), one E4M3 scale per 16 consecutive K elements of every
 * row of A and of B (SA: M x K/16 bytes, SB: N x K/16), and one FP32 scale per
 * tensor (gA, gB):
 *
 *   a(i,k) = e2m1(A[i][k]) * e4m3(SA[i][k/16]) * gA
 *   b(j,k) = e2m1(B[j][k]) * e4m3(SB[j][k/16]) * gB
 *
 * and then the same sums as every other form.  gA, gB are the exact values of
 * the fp32 arguments.
 */
static double nv4_value(const uint8_t* X, const uint8_t* SX, double g, int64_t K, int64_t r,
                        int64_t k) {
    const int64_t idx = r * K + k;
    const uint8_t byte = X[idx / 2];
    return dec_e2m1((idx & 1) ? byte >> 4 : byte & 0xF) * dec_e4m3(SX[r * (K / 16) + k / 16]) * g;
}

int oracle_gemm_nvfp4(const uint8_t* A, const uint8_t* B, const uint8_t* SA, const uint8_t* SB,
                      double gA, double gB, int64_t M, int64_t N, int64_t K, double* ref,
                      double* abssum, int nthreads) {
    if (!A || !B || !SA || !SB || !shape_ok(1, M, N, K) || K % 16 != 0)
        return -1;
    double* a = (double*)malloc((size_t)(M * K > 0 ? M * K : 1) * sizeof(double));
    double* b = (double*)malloc((size_t)(N * K > 0 ? N * K : 1) * sizeof(double));
    if (!a || !b) {
        free(a);
        free(b);
        return -2;
    }
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k)
            a[i * K + k] = nv4_value(A, SA, gA, K, i, k);
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k)
            b[j * K + k] = nv4_value(B, SB, gB, K, j, k);
    int rc = run_rows(a, b, M, N, K, ref, abssum, nthreads);
    free(a);
    free(b);
    return rc;
}

/* Selected entries (ii[t], jj[t]) of the NVFP4 product, one by one. */
int oracle_entries_nvfp4(const uint8_t* A, const uint8_t* B, const uint8_t* SA,
                         const uint8_t* SB, double gA, double gB, int64_t M, int64_t N, int64_t K,
                         const int64_t* ii, const int64_t* jj, int64_t n, double* ref,
                         double* abssum) {
    if (!A || !B || !SA || !SB || !ii || !jj || !shape_ok(1, M, N, K) || K % 16 != 0)
        return -1;
    for (int64_t t = 0; t < n; ++t) {
        const int64_t i = ii[t], j = jj[t];
        if (i < 0 || i >= M || j < 0 || j >= N)
            return -1;
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double prod = nv4_value(A, SA, gA, K, i, k) * nv4_value(B, SB, gB, K, j, k);
            s += prod;
            sa += fabs(prod);
        }
        if (ref)
            ref[t] = s;
        if (abssum)
            abssum[t] = sa;
    }
    return 0;
}
