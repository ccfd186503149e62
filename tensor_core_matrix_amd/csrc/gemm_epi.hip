// Kernel instances and launcher for the product with a C input,
// Out = alpha * (A B^T) + beta * C (float16 / bfloat16 inputs; fp32, bf16 or
// fp16 output).
#include "gemm_kernel.h"

namespace tcm {

template <class Op, typename TOut, int BM, int BN, int OCC, int NSPLIT>
static hipError_t launch_ab(const GemmArgs& a, int grid, hipStream_t st) {
    // swizzle shift 1: 128-byte rows of 64-deep 16-bit slices
    // separate leading dimensions for A and B.  Where one workgroup has the
    // CU and the output is 16-bit, every interior tile without a C input
    // (beta = 0) or an operation stages its output through LDS, alpha
    // applied as the accumulators are staged; edge tiles and calls with a C
    // input or an operation take the alpha/beta epilogue
    constexpr bool epi = OCC == 1 && sizeof(TOut) == 2;
    hipLaunchKernelGGL((tiled_gemm_kernel<Op, TOut, BM, BN, 64, 2, OCC, 1, false, NSPLIT, epi,
                                          false, true, false, false, false>),
                       dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <class Op, typename TOut>
static hipError_t by_variant(int32_t v, const GemmArgs& a, int grid, hipStream_t st) {
    switch (v) {
    case V_T128x256: return launch_ab<Op, TOut, 128, 256, 1, 1>(a, grid, st);
    case V_T128x128: return launch_ab<Op, TOut, 128, 128, 2, 1>(a, grid, st);
    case V_T128x64: return launch_ab<Op, TOut, 128, 64, 3, 1>(a, grid, st);
    default:
        // every 256 x 256 plan runs the default 256 x 256 schedule here
        if (variant_info(v).tile_m == 256 && variant_info(v).elem_bits == 16 &&
            variant_info(v).threads == kThreads)
            return launch_ab<Op, TOut, 256, 256, 1, 3>(a, grid, st);
    }
    return hipErrorInvalidValue;
}

template <class Op>
static hipError_t by_out(int32_t v, int32_t out_dtype, const GemmArgs& a, int grid,
                         hipStream_t st) {
    switch (out_dtype) {
    case 0: return by_variant<Op, _Float16>(v, a, grid, st);
    case 1: return by_variant<Op, __bf16>(v, a, grid, st);
    case 2: return by_variant<Op, float>(v, a, grid, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_epi(int32_t v, int32_t in_dtype, int32_t out_dtype, const GemmArgs& a,
                           int grid, hipStream_t st) {
    if (in_dtype == 1) return by_out<OpBF16>(v, out_dtype, a, grid, st);
    return by_out<OpF16>(v, out_dtype, a, grid, st);
}

}  // namespace tcm
