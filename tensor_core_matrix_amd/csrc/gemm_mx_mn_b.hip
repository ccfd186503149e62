// MXFP8 instances: A K-major, B N-major, with leading dimensions.
#include "gemm_mx_mn.h"

namespace tcm {
template hipError_t launch_gemm_mx_mn<false, true>(int32_t, int32_t, int32_t, const GemmArgs&, int,
                                              hipStream_t);
}  // namespace tcm
