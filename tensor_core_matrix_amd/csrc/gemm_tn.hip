// Kernel instances and launcher for the float16 / bfloat16 TN product.
#include "gemm16.h"
#include "gemm_kernel.h"

namespace tcm {

// The 16-byte chunk XOR of an LDS row uses row bits selected by a shift.  A
// 16-byte fragment read is served 16 lanes (16 consecutive rows) at a time
// across 64 four-byte banks (256 bytes), so the 16 rows of a group must land
// on 16 different 16-byte bank groups: with 128-byte rows (64-deep bf16
// slices) row r covers groups 8 (r % 2) + chunk, and the chunk is XORed with
// (r / 2) % 8; with 64-byte rows (32-deep slices) row r covers groups
// 4 (r % 4) + chunk, and the chunk is XORed with (r / 4) % 4.
template <int BK>
constexpr int swizzle_shift() { return BK == 64 ? 1 : 2; }

// Output staging through LDS is used where the ring leaves room for it: 32
// rows of each wave's output tile per wave, next to the ring.
template <typename TOut, int BM, int BN, int BK, int S>
constexpr bool epilogue_fits() {
    return S * (BM + BN) * BK * 2 + 4 * 32 * (BN / 2) * (int)sizeof(TOut) <= 160 * 1024;
}

template <class Op, typename TOut, int BM, int BN, int BK, int S, int OCC, int NSPLIT = 1>
static hipError_t launch_one(const GemmArgs& a, int grid, hipStream_t st) {
    constexpr bool epi = OCC == 1 && epilogue_fits<TOut, BM, BN, BK, S>();
    hipLaunchKernelGGL(
        (tiled_gemm_kernel<Op, TOut, BM, BN, BK, S, OCC, swizzle_shift<BK>(), false, NSPLIT, epi>),
        dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

// The 16 x 16 x 32 form of each operand type (gemm16.h).
template <class Op> struct op16;
template <> struct op16<OpBF16> { typedef Op16BF16 type; };
template <> struct op16<OpF16> { typedef Op16F16 type; };

template <class Op, typename TOut>
static hipError_t by_variant(int32_t v, const GemmArgs& a, int grid, hipStream_t st) {
    switch (v) {
    case V_T128x256: return launch_one<Op, TOut, 128, 256, 64, 2, 1>(a, grid, st);
    case V_T128x128: return launch_one<Op, TOut, 128, 128, 64, 2, 2>(a, grid, st);
    case V_T128x64: return launch_one<Op, TOut, 128, 64, 64, 2, 3>(a, grid, st);
    case V_T256x256_SPLIT3: return launch_one<Op, TOut, 256, 256, 64, 2, 1, 3>(a, grid, st);
    case V_T256x256_M16:
        hipLaunchKernelGGL((gemm16_kernel<typename op16<Op>::type, TOut>), dim3(grid), dim3(kThreads), 0,
                           st, a);
        return hipGetLastError();
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
