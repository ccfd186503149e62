// Kernel instances and launcher for the MXFP8 (E4M3 + E8M0 per 32) product.
#include "gemm16_mx.h"
#include "gemm_pingpong.h"

namespace tcm {

// LDS rows of a 128-deep fp8 slice are 128 bytes (8 chunks); as for 64-deep
// bf16 slices the chunk is XORed with (row / 2) % 8 so that the 16 rows read
// together by 16 lanes hit 16 different 16-byte bank groups.
constexpr int kSwizzle8 = 1;

template <typename TOut, int BM, int BN, bool WORDS>
static hipError_t launch_one(const GemmArgs& a, int grid, hipStream_t st) {
    constexpr bool epi = 2 * (BM + BN) * 128 + 4 * 32 * (BN / 2) * (int)sizeof(TOut) <= 160 * 1024;
    hipLaunchKernelGGL(
        (tiled_gemm_kernel<OpMXFP8, TOut, BM, BN, 128, 2, 1, kSwizzle8, WORDS, 1, epi>),
        dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <typename TOut, int MODE, int UNIT_K, int S, class Op = OpMXFP8>
static hipError_t launch_pp(const GemmArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL((pingpong_gemm_kernel<Op, TOut, UNIT_K, S, MODE>),
                       dim3(grid), dim3(kPPThreads), 0, st, a);
    return hipGetLastError();
}

// MODE: 0 scale rows read byte by byte, 1 as 32-bit words, 2 as 16-byte pieces
// (the tiled kernels read words in modes 1 and 2).
template <typename TOut, int MODE>
static hipError_t by_variant(int32_t v, const GemmArgs& a, int grid, hipStream_t st) {
    constexpr bool WORDS = MODE >= 1;
    switch (v) {
    case V_MX128x128: return launch_one<TOut, 128, 128, WORDS>(a, grid, st);
    case V_MXPP256_K64S4: return launch_pp<TOut, MODE, 64, 4>(a, grid, st);
    case V_MX4PP256: return launch_pp<TOut, MODE, 128, 4, OpMXFP4>(a, grid, st);
    case V_MX16_256:
        if constexpr (MODE == 2) {
            hipLaunchKernelGGL((gemm16_mx_kernel<TOut>), dim3(grid), dim3(kThreads), 0, st, a);
            return hipGetLastError();
        }
        break;
    case V_MX4_16_256:
        if constexpr (MODE == 2) {
            hipLaunchKernelGGL((gemm16_kernel<Op16MXFP4, TOut>), dim3(grid), dim3(kThreads), 0, st, a);
            return hipGetLastError();
        }
        break;
    }
    return hipErrorInvalidValue;
}

template <typename TOut>
static hipError_t by_mode(int32_t v, int32_t mode, const GemmArgs& a, int grid, hipStream_t st) {
    switch (mode) {
    case 2: return by_variant<TOut, 2>(v, a, grid, st);
    case 1: return by_variant<TOut, 1>(v, a, grid, st);
    default: return by_variant<TOut, 0>(v, a, grid, st);
    }
}

hipError_t launch_gemm_mx(int32_t v, int32_t out_dtype, int32_t scale_mode, const GemmArgs& a,
                          int grid, hipStream_t st) {
    if (out_dtype == 1) return by_mode<__bf16>(v, scale_mode, a, grid, st);
    return by_mode<float>(v, scale_mode, a, grid, st);
}

}  // namespace tcm
