// Host/device shared definitions of libtcm (not part of the public ABI).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace tcm {

constexpr int kThreads = 256;  // four 64-lane waves per workgroup, one per SIMD

// Arguments of one launch of the tiled product kernels.  Sizes are per
// problem; the byte strides step from one batched problem to the next.
struct GemmArgs {
    const void* A;
    const void* B;
    const void* SA;  // E8M0 scales (MX only)
    const void* SB;
    void* C;
    int32_t M, N, K;
    int32_t batch;
    int64_t stride_a, stride_b, stride_c;  // bytes
    int32_t tiles_m, tiles_n;
    int32_t tiles_per_batch;
    int32_t total_tiles;
    int32_t ksteps;   // K slices per tile (at least 1, so K == 0 writes zeros)
    int32_t group_m;  // tile rows per group of the grouped tile order
    // epilogue with a C input (Out = alpha * A B^T + beta * Cin; the kernels
    // built for it only): Cin is M x N of c_dtype (tcm_dtype code), read only
    // when beta != 0
    const void* Cin;
    int64_t stride_cin;  // bytes
    float alpha, beta;
    int32_t c_dtype;
    // Leading dimensions in elements.  lda / ldb: from one stored row of A / B
    // to the next (the 4-wave kernels built for them; the dense instances
    // and the ping-pong kernel take K, and N for ldc).  For an
    // operand stored K-major (the TN form) a row holds K values; stored
    // M-major (N-major for B), a row holds one k of every output row (column).
    // ldc / ldcin: from one row of Out / of the C input to the next.
    int32_t lda, ldb;
    int32_t ldc, ldcin;
    int32_t op;  // per-element epilogue operation (tcm_op code; C-input kernels only)
};

// Kernel variants.  The id is reported by tcm_plan_gemm.  (Ids of variants
// that measured slower and were removed are not reused.)
enum Variant : int32_t {
    V_T128x256 = 1,   // 128x256x64, 2-stage ring
    V_T128x128 = 2,   // 128x128x64, 2-stage ring, 2 workgroups per CU
    V_T128x64 = 3,    // 128x64x64, 2-stage ring, 3 workgroups per CU
    V_MX128x128 = 11,       // MXFP8 128x128x128, 2-stage ring
    V_MXPP256_K64S4 = 14,   // MXFP8 256x256x64 ping-pong, 4-stage ring
    V_T256x256_SPLIT3 = 19, // 256x256x64, 2-stage ring, copies split over 3 K steps (6/5/5)
    V_MX4PP256 = 20,        // MXFP4 256x256x128 ping-pong, 4-stage ring
    V_MX6PP256 = 21,        // MXFP6 256x256x64 ping-pong, 4-stage ring, rows stored row after row
    V_NV4_256 = 22,         // NVFP4 256x256x64, dequantizing register-staged copies, fp16 MFMA
    V_NV4_128 = 23,         // NVFP4 128x128x64, the same
    V_NV4W_256 = 24,        // V_NV4_256 with a row's scales of four slices in one load
    V_NV4W_128 = 25,        // V_NV4_128, the same
    V_MX256x128 = 26,       // MXFP8 256x128x128, 2-stage ring (arrangements and leading dimensions)
    V_MX6PP256_K128 = 27,   // MXFP6 ping-pong, 128-deep units (96-byte rows), ring of 3
    V_T256x256_M16 = 28,    // 256x256x64 on the 16x16x32 MFMA, 2-stage ring (gemm16.h)
    V_MX16_256 = 31,        // MXFP8 256x256x128 on the 16x16x128 scaled MFMA, scale chunks by DMA (gemm16_mx.h)
    V_MX4_16_256 = 32,      // MXFP4 256x256x256 on the 16x16x128 scaled MFMA, scale chunks by DMA (gemm16.h)
    V_NV4_16_256 = 34,      // NVFP4 256x256x256, E2M1 rows by DMA, converted per fragment for the 16x16x32 fp16 MFMA (gemm16_nv4.h)
    V_MX6_16_256 = 36,      // MXFP6 256x256x128 on the 16x16x128 scaled MFMA, 96-byte rows in 128-byte LDS rows (gemm16_mx.h)
};

struct VariantInfo {
    int32_t tile_m, tile_n, tile_k, stages, occupancy;
    int32_t elem_bits;  // 16 f16/bf16, 8 MXFP8, 6 MXFP6, 4 MXFP4
    int32_t threads;
};

VariantInfo variant_info(int32_t v);

// Launchers (one per translation unit).  dtype codes follow tcm_dtype.
hipError_t launch_gemm_tn(int32_t variant, int32_t in_dtype, int32_t out_dtype, const GemmArgs& a,
                          int grid, hipStream_t stream);
// scale_mode: how E8M0 rows may be read -- 0 bytes, 1 32-bit words (K % 128 == 0,
// word-aligned arrays), 2 16-byte pieces (K % 512 == 0, 16-byte-aligned arrays).
hipError_t launch_gemm_epi(int32_t variant, int32_t in_dtype, int32_t out_dtype, const GemmArgs& a,
                           int grid, hipStream_t stream);
// A stored M-major (A_MN) and/or B stored N-major (B_MN), C-input epilogue;
// variants V_T256x256_SPLIT3 and V_T128x128 only.  One translation unit per
// arrangement.
template <bool A_MN, bool B_MN>
hipError_t launch_gemm_mn(int32_t variant, int32_t in_dtype, int32_t out_dtype, const GemmArgs& a,
                          int grid, hipStream_t stream);
hipError_t launch_gemm_mx(int32_t variant, int32_t out_dtype, int32_t scale_mode, const GemmArgs& a,
                          int grid, hipStream_t stream);
// MXFP8 with an M-major A (A_MN) and/or N-major B (B_MN) and leading
// dimensions (lda, ldb, ldc); variants V_MX256x128 and V_MX128x128.  One translation
// unit per arrangement.
template <bool A_MN, bool B_MN>
hipError_t launch_gemm_mx_mn(int32_t variant, int32_t out_dtype, int32_t scale_mode,
                             const GemmArgs& a, int grid, hipStream_t stream);
// NVFP4 (variants V_NV4_*): GemmArgs.SA/SB hold the E4M3 block scales and
// alpha the product of the two tensor scales.
hipError_t launch_gemm_nv4(int32_t variant, int32_t out_dtype, const GemmArgs& a, int grid,
                           hipStream_t stream);
// MXFP6; elem_dtype is the tcm_dtype of both operands' elements (E2M3 or E3M2).
hipError_t launch_gemm_mx6(int32_t variant, int32_t out_dtype, int32_t scale_mode,
                           int32_t elem_dtype, const GemmArgs& a, int grid, hipStream_t stream);

}  // namespace tcm
