// Kernel instances and launcher for the NVFP4 product (E2M1 + E4M3 per 16 +
// fp32 per tensor): register-staged copies that dequantize into fp16 LDS
// tiles, the fp16 MFMA, and the C-input epilogue (alpha = the two tensor
// scales' product).
#include "gemm16_nv4.h"

namespace tcm {

template <typename TOut, int BM, int BN, int OCC, int NSPLIT, bool WIDE>
static hipError_t launch_nv4(const GemmArgs& a, int grid, hipStream_t st) {
    // swizzle shift 1: 128-byte fp16 rows of 64-deep slices; a 16-bit output
    // is staged through LDS where one workgroup has the CU
    constexpr bool epi = OCC == 1 && sizeof(TOut) == 2;
    hipLaunchKernelGGL((tiled_gemm_kernel<OpNVFP4<WIDE>, TOut, BM, BN, 64, 2, OCC, 1, false, NSPLIT, epi,
                                          true, true, false, false, false>),
                       dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <typename TOut>
static hipError_t by_variant(int32_t v, const GemmArgs& a, int grid, hipStream_t st) {
    switch (v) {
    case V_NV4_256: return launch_nv4<TOut, 256, 256, 1, 2, false>(a, grid, st);
    case V_NV4_128: return launch_nv4<TOut, 128, 128, 2, 1, false>(a, grid, st);
    case V_NV4W_256: return launch_nv4<TOut, 256, 256, 1, 2, true>(a, grid, st);
    case V_NV4W_128: return launch_nv4<TOut, 128, 128, 2, 1, true>(a, grid, st);
    case V_NV4_16_256:
        hipLaunchKernelGGL((gemm16_nv4_kernel<TOut>), dim3(grid), dim3(kThreads), 0, st, a);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_nv4(int32_t v, int32_t out_dtype, const GemmArgs& a, int grid,
                           hipStream_t st) {
    switch (out_dtype) {
    case 0: return by_variant<_Float16>(v, a, grid, st);
    case 1: return by_variant<__bf16>(v, a, grid, st);
    case 2: return by_variant<float>(v, a, grid, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace tcm
