// Kernel instances and launcher for the MXFP8 (E4M3 + E8M0 per 32) product.
#include "gemm_pingpong.h"

namespace tcm {

// LDS rows of a 128-deep fp8 slice are 128 bytes (8 chunks); as for 64-deep
// bf16 slices the chunk is XORed with (row / 2) % 8 so that the 16 rows read
// together by 16 lanes hit 16 different 16-byte bank groups.
constexpr int kSwizzle8 = 1;

template <typename TOut, int BM, int BN, bool WORDS, int NSPLIT = 1>
static hipError_t launch_one(const GemmArgs& a, int grid, hipStream_t st) {
    constexpr bool epi = 2 * (BM + BN) * 128 + 4 * 32 * (BN / 2) * (int)sizeof(TOut) <= 160 * 1024;
    hipLaunchKernelGGL(
        (tiled_gemm_kernel<OpMXFP8, TOut, BM, BN, 128, 2, 1, kSwizzle8, WORDS, NSPLIT, epi>),
        dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <typename TOut, bool WORDS, int UNIT_K, int S>
static hipError_t launch_pp(const GemmArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL((pingpong_gemm_kernel<OpMXFP8, TOut, UNIT_K, S, WORDS>), dim3(grid),
                       dim3(kPPThreads), 0, st, a);
    return hipGetLastError();
}

template <typename TOut, bool WORDS>
static hipError_t by_variant(int32_t v, const GemmArgs& a, int grid, hipStream_t st) {
    switch (v) {
    case V_MX256x256: return launch_one<TOut, 256, 256, WORDS>(a, grid, st);
    case V_MX128x128: return launch_one<TOut, 128, 128, WORDS>(a, grid, st);
    case V_MX256x256_SPLIT2: return launch_one<TOut, 256, 256, WORDS, 2>(a, grid, st);
    case V_MXPP256: return launch_pp<TOut, WORDS, 128, 2>(a, grid, st);
    case V_MXPP256_K64S4: return launch_pp<TOut, WORDS, 64, 4>(a, grid, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_mx(int32_t v, int32_t out_dtype, bool scale_words, const GemmArgs& a,
                          int grid, hipStream_t st) {
    if (out_dtype == 1)
        return scale_words ? by_variant<__bf16, true>(v, a, grid, st)
                           : by_variant<__bf16, false>(v, a, grid, st);
    return scale_words ? by_variant<float, true>(v, a, grid, st)
                       : by_variant<float, false>(v, a, grid, st);
}

}  // namespace tcm
