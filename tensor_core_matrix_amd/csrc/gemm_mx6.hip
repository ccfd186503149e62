// Kernel instances and launcher for the MXFP6 (E2M3 or E3M2 + E8M0 per 32)
// product: the ping-pong kernel with 64- or 128-deep units, and the 16 x 16
// x 128 kernel of gemm16_mx.h where scales come as 16-byte pieces.
#include "gemm16_mx.h"
#include "gemm_pingpong.h"

namespace tcm {

template <typename TOut, int MODE, int FMT, int UNIT_K, int S>
static hipError_t launch6(const GemmArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL((pingpong_gemm_kernel<OpMXFP6<FMT>, TOut, UNIT_K, S, MODE>),
                       dim3(grid), dim3(kPPThreads), 0, st, a);
    return hipGetLastError();
}

template <typename TOut, int FMT, int UNIT_K, int S>
static hipError_t by_mode(int32_t mode, const GemmArgs& a, int grid, hipStream_t st) {
    switch (mode) {
    case 2: return launch6<TOut, 2, FMT, UNIT_K, S>(a, grid, st);
    case 1: return launch6<TOut, 1, FMT, UNIT_K, S>(a, grid, st);
    default: return launch6<TOut, 0, FMT, UNIT_K, S>(a, grid, st);
    }
}

template <typename TOut, int FMT>
static hipError_t by_variant(int32_t v, int32_t mode, const GemmArgs& a, int grid, hipStream_t st) {
    switch (v) {
    case V_MX6PP256: return by_mode<TOut, FMT, 64, 4>(mode, a, grid, st);
    case V_MX6PP256_K128: return by_mode<TOut, FMT, 128, 3>(mode, a, grid, st);
    case V_MX6_16_256:
        if (mode == 2) {
            hipLaunchKernelGGL((gemm16_mx_kernel<TOut, FMT>), dim3(grid), dim3(kThreads), 0, st, a);
            return hipGetLastError();
        }
        break;
    }
    return hipErrorInvalidValue;
}

// elem_dtype: tcm_dtype code 6 (E2M3, format code 2) or 7 (E3M2, format code 3)
hipError_t launch_gemm_mx6(int32_t v, int32_t out_dtype, int32_t scale_mode, int32_t elem_dtype,
                           const GemmArgs& a, int grid, hipStream_t st) {
    const bool bf = out_dtype == 1;
    if (elem_dtype == 7)
        return bf ? by_variant<__bf16, 3>(v, scale_mode, a, grid, st)
                  : by_variant<float, 3>(v, scale_mode, a, grid, st);
    return bf ? by_variant<__bf16, 2>(v, scale_mode, a, grid, st)
              : by_variant<float, 2>(v, scale_mode, a, grid, st);
}

}  // namespace tcm
