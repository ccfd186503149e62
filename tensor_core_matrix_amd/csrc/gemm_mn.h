// Launcher of the product with an M-major A and/or an N-major B (16-bit
// inputs; C-input epilogue; fp32, bf16 or fp16 output).  Each arrangement is
// instantiated in its own translation unit so that they compile in parallel.
#pragma once

#include "gemm_kernel.h"

namespace tcm {

template <class Op, typename TOut, int BM, int BN, int OCC, int NSPLIT, bool A_MN, bool B_MN>
static hipError_t launch_mn_one(const GemmArgs& a, int grid, hipStream_t st) {
    // swizzle shift 1: 128-byte rows of the K-major operand's 64-deep slices
    // where one workgroup has the CU and the output is 16-bit, every
    // interior tile without a C input (beta = 0) or an operation stages its
    // output through LDS, alpha applied as the accumulators are staged;
    // edge tiles and calls with a C input or an operation take the
    // alpha/beta epilogue
    constexpr bool epi = OCC == 1 && sizeof(TOut) == 2;
    hipLaunchKernelGGL((tiled_gemm_kernel<Op, TOut, BM, BN, 64, 2, OCC, 1, false, NSPLIT, epi,
                                          false, true, A_MN, B_MN, false>),
                       dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <class Op, typename TOut, bool A_MN, bool B_MN>
static hipError_t launch_mn_tile(int32_t v, const GemmArgs& a, int grid, hipStream_t st) {
    switch (v) {
    case V_T256x256_SPLIT3: return launch_mn_one<Op, TOut, 256, 256, 1, 3, A_MN, B_MN>(a, grid, st);
    case V_T128x128: return launch_mn_one<Op, TOut, 128, 128, 2, 1, A_MN, B_MN>(a, grid, st);
    }
    return hipErrorInvalidValue;
}

template <bool A_MN, bool B_MN>
hipError_t launch_gemm_mn(int32_t v, int32_t in_dtype, int32_t out_dtype, const GemmArgs& a,
                          int grid, hipStream_t st) {
    const bool bf = in_dtype == 1;
    switch (out_dtype) {
    case 0:
        return bf ? launch_mn_tile<OpBF16, _Float16, A_MN, B_MN>(v, a, grid, st)
                  : launch_mn_tile<OpF16, _Float16, A_MN, B_MN>(v, a, grid, st);
    case 1:
        return bf ? launch_mn_tile<OpBF16, __bf16, A_MN, B_MN>(v, a, grid, st)
                  : launch_mn_tile<OpF16, __bf16, A_MN, B_MN>(v, a, grid, st);
    case 2:
        return bf ? launch_mn_tile<OpBF16, float, A_MN, B_MN>(v, a, grid, st)
                  : launch_mn_tile<OpF16, float, A_MN, B_MN>(v, a, grid, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace tcm
