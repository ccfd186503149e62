// MXFP8 (E4M3 + E8M0 per 32) with operands in either arrangement and
// leading dimensions: the 4-wave kernel's 256 x 128 x 128 and 128 x 128 x 128
// tiles (at 256 x 256 the 32-byte MX fragments push the kernel past its
// registers), an M-major A
// and/or N-major B staged k row by k row and read with ds_read_b64_tr_b8
// (A_MN / B_MN in gemm_kernel.h).  One translation unit per arrangement.
#pragma once
#include "gemm_pingpong.h"

namespace tcm {

// LDS rows of a K-major 128-deep fp8 slice are 128 bytes (8 chunks), chunk
// XORed with (row / 2) % 8, as for the TN MX kernels.
constexpr int kMxMnSwizzle = 1;

template <typename TOut, int BM, int BN, bool A_MN, bool B_MN, bool WORDS>
static hipError_t launch_mx_mn_one(const GemmArgs& a, int grid, hipStream_t st) {
    constexpr bool epi = 2 * (BM + BN) * 128 + 4 * 32 * (BN / 2) * (int)sizeof(TOut) <= 160 * 1024;
    hipLaunchKernelGGL((tiled_gemm_kernel<OpMXFP8, TOut, BM, BN, 128, 2, 1, kMxMnSwizzle, WORDS, 1,
                                          epi, false, false, A_MN, B_MN, false>),
                       dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <typename TOut, int BM, int BN, bool A_MN, bool B_MN>
static hipError_t by_scale_mode(int32_t scale_mode, const GemmArgs& a, int grid, hipStream_t st) {
    return scale_mode >= 1 ? launch_mx_mn_one<TOut, BM, BN, A_MN, B_MN, true>(a, grid, st)
                           : launch_mx_mn_one<TOut, BM, BN, A_MN, B_MN, false>(a, grid, st);
}

// The ping-pong kernel (eight waves, ring of four 64-deep units) with an
// M/N-major operand; scale_mode as for the TN MX kernels (0 bytes, 1 words,
// 2 16-byte chunks).
template <typename TOut, bool A_MN, bool B_MN>
static hipError_t launch_mx_pp_mn(int32_t scale_mode, const GemmArgs& a, int grid, hipStream_t st) {
    if constexpr (A_MN || B_MN) {
        switch (scale_mode) {
        case 2:
            hipLaunchKernelGGL((pingpong_gemm_kernel<OpMXFP8, TOut, 64, 4, 2, A_MN, B_MN>),
                               dim3(grid), dim3(kPPThreads), 0, st, a);
            break;
        case 1:
            hipLaunchKernelGGL((pingpong_gemm_kernel<OpMXFP8, TOut, 64, 4, 1, A_MN, B_MN>),
                               dim3(grid), dim3(kPPThreads), 0, st, a);
            break;
        default:
            hipLaunchKernelGGL((pingpong_gemm_kernel<OpMXFP8, TOut, 64, 4, 0, A_MN, B_MN>),
                               dim3(grid), dim3(kPPThreads), 0, st, a);
        }
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;  // both operands K-major: the 4-wave kernels
    }
}

// scale_mode >= 1: each fragment row's scales of a slice read as one word
template <bool A_MN, bool B_MN>
hipError_t launch_gemm_mx_mn(int32_t variant, int32_t out_dtype, int32_t scale_mode,
                             const GemmArgs& a, int grid, hipStream_t st) {
    const bool bf = out_dtype == 1;
    switch (variant) {
    case V_MXPP256_K64S4:
        return bf ? launch_mx_pp_mn<__bf16, A_MN, B_MN>(scale_mode, a, grid, st)
                  : launch_mx_pp_mn<float, A_MN, B_MN>(scale_mode, a, grid, st);
    case V_MX256x128:
        return bf ? by_scale_mode<__bf16, 256, 128, A_MN, B_MN>(scale_mode, a, grid, st)
                  : by_scale_mode<float, 256, 128, A_MN, B_MN>(scale_mode, a, grid, st);
    case V_MX128x128:
        return bf ? by_scale_mode<__bf16, 128, 128, A_MN, B_MN>(scale_mode, a, grid, st)
                  : by_scale_mode<float, 128, 128, A_MN, B_MN>(scale_mode, a, grid, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace tcm
