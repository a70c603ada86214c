// mx_internal.h -- launchers shared between the C-ABI layer and the kernels.
// Arguments have been validated by the caller (mx_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

struct QuantArgs {
  const void* x;
  int64_t rows, cols, ld_bytes;  // source pitch in bytes
  int src, fmt, round;
  bool hadamard;
  uint32_t signs;
  uint64_t seed, counter_offset;
  uint8_t* q_row;
  uint8_t* s_row;
  uint8_t* q_colt;
  uint8_t* s_colt;
};

// Row-wise layout only.
hipError_t launch_quant_rows(const QuantArgs& a, hipStream_t st);
// Column-wise layout, optionally fused with the row-wise one (dual).
hipError_t launch_quant_tiles(const QuantArgs& a, bool with_rows, hipStream_t st);
hipError_t launch_dequant(const void* q, const uint8_t* s, int fmt, int64_t rows, int64_t cols,
                          float* y, hipStream_t st);
// out_fmt < 0: fp32 C (c, ldc).  GEMM_OUT_BF16: bf16 C at out_q, row pitch
// ldc elements.  Otherwise C goes out row-wise in MX format out_fmt (E4M3,
// E5M2, E2M1) to out_q / out_s; only the staged kernel does that
// (hipErrorNotSupported otherwise).
constexpr int GEMM_OUT_BF16 = 16;
hipError_t launch_gemm(const void* a_q, const uint8_t* a_s, int a_fmt, const void* b_q,
                       const uint8_t* b_s, int b_fmt, int64_t M, int64_t N, int64_t K, float* c,
                       int64_t ldc, int out_fmt, uint8_t* out_q, uint8_t* out_s, hipStream_t st);

// One GEMM call as the kernels' launchers take it (K already a multiple of 32).
struct GemmCall {
  const void* aq;
  const uint8_t* as;
  const void* bq;
  const uint8_t* bs;
  int64_t M, N, K;
  float* c;
  int64_t ldc;
  int out_fmt;
  uint8_t* out_q;
  uint8_t* out_s;
  hipStream_t st;
};
// Launcher of one operand-format pair (explicitly instantiated per pair by
// the build, from mx_gemm_kernels.hpp).
template <int FA, int FB>
hipError_t gemm_launch(const GemmCall& gc);

inline int elem_bits(int fmt) { return fmt == 2 || fmt == 3 ? 6 : (fmt == 4 ? 4 : 8); }

}  // namespace mx
