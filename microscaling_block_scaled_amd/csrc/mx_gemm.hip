// mx_gemm.hip -- dispatch of an MX GEMM call to the launcher of its operand
// formats (the kernels are in mx_gemm_kernels.hpp; the build instantiates
// gemm_launch once per format pair, each in a unit of its own).
#include "mx_device.hpp"
#include "mx_internal.h"

namespace mx {

hipError_t launch_gemm(const void* aq, const uint8_t* as, int fa, const void* bq,
                       const uint8_t* bs, int fb, int64_t M, int64_t N, int64_t K, float* c,
                       int64_t ldc, int out_fmt, uint8_t* out_q, uint8_t* out_s, hipStream_t st) {
  const GemmCall gc{aq, as, bq, bs, M, N, K, c, ldc, out_fmt, out_q, out_s, st};
  if (fa == INT8 && fb == INT8) return gemm_launch<INT8, INT8>(gc);
#define MX_G(A, B) \
  if (fa == A && fb == B) return gemm_launch<A, B>(gc);
#define MX_GA(A) MX_G(A, E4M3) MX_G(A, E5M2) MX_G(A, E2M3) MX_G(A, E3M2) MX_G(A, E2M1)
  MX_GA(E4M3) MX_GA(E5M2) MX_GA(E2M3) MX_GA(E3M2) MX_GA(E2M1)
#undef MX_GA
#undef MX_G
  return hipErrorInvalidValue;
}

}  // namespace mx
