// mx_dequant.hip -- v_i = X * P_i for packed MX tensors ("Microscaling Data
// Formats for Deep Learning", summary section 2: block semantics, NaN scale).
//
// One lane decodes 8 consecutive elements of a row (one 8/6/4-byte packed
// chunk) and writes 32 bytes of fp32.  Element values are built exactly from
// their bit fields and scaled with ldexp, so the result is exact unless it
// overflows fp32 (Inf).
#include "mx_device.hpp"
#include "mx_internal.h"

namespace mx {

template <int F>
__device__ __forceinline__ float decode(uint32_t c) {
  using T = Fmt<F>;
  if (F == INT8) return (float)(int32_t)(int8_t)(uint8_t)c * 0.015625f;
  constexpr int ebits = T::bits - 1 - T::mbits;
  const uint32_t s = (c >> (T::bits - 1)) & 1u;
  const uint32_t e = (c >> T::mbits) & ((1u << ebits) - 1u);
  const uint32_t m = c & ((1u << T::mbits) - 1u);
  float v;
  if (F == E4M3 && e == 15 && m == 7) {
    v = __builtin_nanf("");
  } else if (F == E5M2 && e == 31) {
    v = m == 0 ? __builtin_inff() : __builtin_nanf("");
  } else if (e == 0) {  // subnormal: m * 2^(emin - mbits)
    v = (float)m * __builtin_bit_cast(float, (uint32_t)(127 + T::emin - T::mbits) << 23);
  } else {
    v = __builtin_bit_cast(float, ((e - T::bias + 127) << 23) | (m << (23 - T::mbits)));
  }
  return s ? -v : v;
}

template <int F>
__device__ __forceinline__ void unpack8(const uint8_t* row, int64_t c, uint32_t out[8]) {
  if (Fmt<F>::bits == 8) {
    const uint2 t = *(const uint2*)(row + 8 * c);
#pragma unroll
    for (int k = 0; k < 4; k++) {
      out[k] = (t.x >> (8 * k)) & 0xFFu;
      out[k + 4] = (t.y >> (8 * k)) & 0xFFu;
    }
  } else if (Fmt<F>::bits == 4) {
    const uint32_t t = *(const uint32_t*)(row + 4 * c);
#pragma unroll
    for (int k = 0; k < 8; k++) out[k] = (t >> (4 * k)) & 0xFu;
  } else {
    const uint8_t* p = row + 6 * c;
    uint64_t t;
    if ((c & 1) == 0)
      t = (uint64_t)(*(const uint32_t*)p) | ((uint64_t)(*(const uint16_t*)(p + 4)) << 32);
    else
      t = (uint64_t)(*(const uint16_t*)p) | ((uint64_t)(*(const uint32_t*)(p + 2)) << 16);
#pragma unroll
    for (int k = 0; k < 8; k++) out[k] = (uint32_t)(t >> (6 * k)) & 0x3Fu;
  }
}

// q holds rows of cols padded to whole blocks (cp elements); y is [rows x cols]
// and the padded positions are dropped.
template <int F>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ q,
                                                 const uint8_t* __restrict__ s, int64_t rows,
                                                 int64_t cols, float* __restrict__ y) {
  const int64_t cp = (cols + 31) / 32 * 32;
  const int64_t cpr = (cols + 7) >> 3;  // chunks of 8 holding at least one element
  const int64_t n = rows * cpr;
  const int64_t pitch = cp * Fmt<F>::bits / 8;
  const bool vec = (cols & 3) == 0;     // rows of y start 16-byte aligned
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / cpr, c = i - r * cpr;
    const uint32_t sc = s[r * (cp >> 5) + (c >> 2)];
    uint32_t codes[8];
    unpack8<F>(q + r * pitch, c, codes);
    float o[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const float v = decode<F>(codes[k]);
      o[k] = sc == 0xFFu ? __builtin_nanf("") : __builtin_amdgcn_ldexpf(v, (int)sc - 127);
    }
    float* yr = y + r * cols + 8 * c;
    if (vec && 8 * c + 8 <= cols) {
      float4* dst = (float4*)yr;
      dst[0] = make_float4(o[0], o[1], o[2], o[3]);
      dst[1] = make_float4(o[4], o[5], o[6], o[7]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; k++)
        if (8 * c + k < cols) yr[k] = o[k];
    }
  }
}

hipError_t launch_dequant(const void* q, const uint8_t* s, int fmt, int64_t rows, int64_t cols,
                          float* y, hipStream_t st) {
  const int64_t n = rows * ((cols + 7) / 8);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const dim3 g((unsigned)blocks), b(256);
  const uint8_t* qq = (const uint8_t*)q;
  switch (fmt) {
    case E4M3: hipLaunchKernelGGL(k_dequant<E4M3>, g, b, 0, st, qq, s, rows, cols, y); break;
    case E5M2: hipLaunchKernelGGL(k_dequant<E5M2>, g, b, 0, st, qq, s, rows, cols, y); break;
    case E2M3: hipLaunchKernelGGL(k_dequant<E2M3>, g, b, 0, st, qq, s, rows, cols, y); break;
    case E3M2: hipLaunchKernelGGL(k_dequant<E3M2>, g, b, 0, st, qq, s, rows, cols, y); break;
    case E2M1: hipLaunchKernelGGL(k_dequant<E2M1>, g, b, 0, st, qq, s, rows, cols, y); break;
    default: hipLaunchKernelGGL(k_dequant<INT8>, g, b, 0, st, qq, s, rows, cols, y); break;
  }
  return hipGetLastError();
}

}  // namespace mx
