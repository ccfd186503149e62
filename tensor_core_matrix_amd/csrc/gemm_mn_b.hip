// Kernel instances: K-major A, N-major B.
#include "gemm_mn.h"

namespace tcm {
template hipError_t launch_gemm_mn<false, true>(int32_t, int32_t, int32_t, const GemmArgs&, int,
                                              hipStream_t);
}  // namespace tcm
