// Kernel instances and launcher for the float16 / bfloat16 TN product.
#include "gemm_kernel.h"

namespace tcm {

// LDS rows of a 64-deep bf16 slice are 128 bytes (8 chunks); the chunk XOR
// uses row bits selected by this shift.
constexpr int kSwizzle16 = 0;

template <class Op, typename TOut, int BM, int BN, int BK, int S, int OCC>
static hipError_t launch_one(const GemmArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL((tiled_gemm_kernel<Op, TOut, BM, BN, BK, S, OCC, kSwizzle16>), dim3(grid),
                       dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <class Op, typename TOut>
static hipError_t by_variant(int32_t v, const GemmArgs& a, int grid, hipStream_t st) {
    switch (v) {
    case V_T256x256: return launch_one<Op, TOut, 256, 256, 64, 2, 1>(a, grid, st);
    case V_T128x256: return launch_one<Op, TOut, 128, 256, 64, 2, 1>(a, grid, st);
    case V_T128x128: return launch_one<Op, TOut, 128, 128, 64, 2, 2>(a, grid, st);
    case V_T128x64: return launch_one<Op, TOut, 128, 64, 64, 2, 3>(a, grid, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_tn(int32_t v, int32_t in_dtype, int32_t out_dtype, const GemmArgs& a,
                          int grid, hipStream_t st) {
    const bool out_bf16 = out_dtype == 1;
    if (in_dtype == 1)
        return out_bf16 ? by_variant<OpBF16, __bf16>(v, a, grid, st)
                        : by_variant<OpBF16, float>(v, a, grid, st);
    if (in_dtype == 0)
        return out_bf16 ? by_variant<OpF16, __bf16>(v, a, grid, st)
                        : by_variant<OpF16, float>(v, a, grid, st);
    return hipErrorInvalidValue;
}

}  // namespace tcm
