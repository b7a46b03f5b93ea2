// GEMM kernels for A E5M2, B E5M2.
#include "gemm_impl.h"

namespace mxg {
template hipError_t launch_gemm_fmt<kE5M2, kE5M2>(int, bool, const GemmArgs&, hipStream_t);
}  // namespace mxg
