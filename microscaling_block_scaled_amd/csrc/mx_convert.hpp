// mx_convert.hpp -- conversion of 8 (or 32) elements of one MX block to packed
// element codes for gfx950: the exact integer conversion (cvt_exact, in
// mx_device.hpp) and the hardware scaled conversions where they were checked
// bit for bit against the definition (Algorithm 1 of "Microscaling Data
// Formats for Deep Learning", summary section 3).  Shared by the quantizers
// and the GEMM's MX-output epilogue.
#pragma once

#include <type_traits>

#include "mx_device.hpp"

namespace mx {

typedef short v2s __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// conversion of 8 elements of one block to packed codes
// ---------------------------------------------------------------------------
// Packed result of 8 elements: FP8 / INT8 8 bytes in w[0..1]; FP6 48 bits (w[0]
// then the low 16 bits of w[1]); FP4 32 bits in w[0].
struct Pack8 { uint32_t w[2]; };

// gfx950's scaled conversions divide by the scale and round to nearest even.
// For E4M3, E5M2 and E2M1 they agree bit for bit with the definition on every
// finite non-subnormal input, except that FP8 overflow gives the NaN / Inf code
// instead of saturating; fix_sat repairs that.  Used only for scale codes at
// which fp32-subnormal inputs round to zero anyway (DazFree), so no flush is
// needed first.
template <int F>
__device__ __forceinline__ uint32_t fix_sat(uint32_t r) {
  if (F == E4M3) {  // 0x7F / 0xFF (NaN) -> 0x7E / 0xFE
    const uint32_t t = r & 0x7F7F7F7Fu;
    return r - (((t + 0x01010101u) & 0x80808080u) >> 7);
  } else {  // E5M2: 0x7C / 0xFC (Inf) -> 0x7B / 0xFB
    const uint32_t t = (r & 0x7F7F7F7Fu) ^ 0x7C7C7C7Cu;
    const uint32_t nz = (((t & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | t) & 0x80808080u;
    return r - ((~nz & 0x80808080u) >> 7);
  }
}

template <int F>
__device__ __forceinline__ Pack8 hw_convert8(const uint32_t v[8], uint32_t code) {
  const float S = __builtin_bit_cast(float, code << 23);  // 2^(code - 127), code >= 1
  float f[8];
#pragma unroll
  for (int k = 0; k < 8; k++) f[k] = __builtin_bit_cast(float, v[k]);
  Pack8 o;
  if (F == E4M3 || F == E5M2) {
#pragma unroll
    for (int h = 0; h < 2; h++) {
      v2s t = {0, 0};
      if (F == E4M3) {
        t = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(t, f[4 * h], f[4 * h + 1], S, false);
        t = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(t, f[4 * h + 2], f[4 * h + 3], S, true);
      } else {
        t = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(t, f[4 * h], f[4 * h + 1], S, false);
        t = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(t, f[4 * h + 2], f[4 * h + 3], S, true);
      }
      o.w[h] = fix_sat<F>(__builtin_bit_cast(uint32_t, t));
    }
  } else {  // E2M1: saturates in hardware
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, f[0], f[1], S, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, f[2], f[3], S, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, f[4], f[5], S, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, f[6], f[7], S, 3);
    o.w[0] = r;
    o.w[1] = 0;
  }
  return o;
}

// The same conversion of 8 bf16 elements held packed in raw[4] (element 2i in
// the low half of raw[i]), through the packed-bf16 form of the instructions;
// bf16 widens to fp32 exactly, so the codes are the same.
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
template <int F>
__device__ __forceinline__ Pack8 hw_convert8_bf16(const uint32_t raw[4], uint32_t code) {
  const float S = __builtin_bit_cast(float, code << 23);
  Pack8 o;
  if (F == E4M3 || F == E5M2) {
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const v2bf a = __builtin_bit_cast(v2bf, raw[2 * h]), b = __builtin_bit_cast(v2bf, raw[2 * h + 1]);
      v2s t = {0, 0};
      if (F == E4M3) {
        t = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(t, a, S, false);
        t = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(t, b, S, true);
      } else {
        t = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(t, a, S, false);
        t = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(t, b, S, true);
      }
      o.w[h] = fix_sat<F>(__builtin_bit_cast(uint32_t, t));
    }
  } else {  // E2M1
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf, raw[0]), S, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf, raw[1]), S, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf, raw[2]), S, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf, raw[3]), S, 3);
    o.w[0] = r;
    o.w[1] = 0;
  }
  return o;
}

// Formats with a hardware conversion that matches the definition (round to
// nearest even only).
template <int F, bool SR> struct HwPath {
  static constexpr bool value = !SR && (F == E4M3 || F == E5M2 || F == E2M1);
};
// ... and those whose hardware conversion takes a whole block of 32 bf16
// elements at once (FP6, also checked bit for bit against the definition).
template <int F, bool SR> struct HwPath32 {
  static constexpr bool value = HwPath<F, SR>::value || (!SR && (F == E2M3 || F == E3M2));
};

// FP6 codes of a whole block of 32 bf16 elements held packed in pr[16]
// (element 2i in the low half of pr[i]): one 32-element conversion, whose
// 24-byte little-endian bit stream is split into the Pack8 groups.
typedef uint32_t v16u __attribute__((ext_vector_type(16)));
typedef __bf16 v32bf __attribute__((ext_vector_type(32)));
typedef int v6i __attribute__((ext_vector_type(6)));
template <int F>
__device__ __forceinline__ void hw_convert32_bf16_fp6(const uint32_t pr[16], uint32_t code, Pack8 o[4]) {
  const float S = __builtin_bit_cast(float, code << 23);
  v16u t;
#pragma unroll
  for (int i = 0; i < 16; i++) t[i] = pr[i];
  const v32bf in = __builtin_bit_cast(v32bf, t);
  v6i r;
  if (F == E2M3)
    r = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(in, S);
  else
    r = __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(in, S);
  const uint32_t d0 = (uint32_t)r[0], d1 = (uint32_t)r[1], d2 = (uint32_t)r[2];
  const uint32_t d3 = (uint32_t)r[3], d4 = (uint32_t)r[4], d5 = (uint32_t)r[5];
  o[0].w[0] = d0;                      o[0].w[1] = d1 & 0xFFFFu;
  o[1].w[0] = (d1 >> 16) | (d2 << 16); o[1].w[1] = d2 >> 16;
  o[2].w[0] = d3;                      o[2].w[1] = d4 & 0xFFFFu;
  o[3].w[0] = (d4 >> 16) | (d5 << 16); o[3].w[1] = d5 >> 16;
}
// Whether a block with scale `code` can take the hardware conversion.
template <int F>
__device__ __forceinline__ bool hw_ok(uint32_t code) {
  return code >= (uint32_t)DazFree<F>::value && code != 0xFFu;
}

// Largest magnitude of the bf16 pairs in w[0 .. n-1], per half: packed 16-bit
// unsigned max of the sign-cleared pairs (a magnitude compare for bf16).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

template <int F>
__device__ __forceinline__ Pack8 pack8(const uint32_t c[8]) {
  Pack8 o;
  if (Fmt<F>::bits == 8) {
    o.w[0] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    o.w[1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
  } else if (Fmt<F>::bits == 4) {
    uint32_t r = 0;
#pragma unroll
    for (int k = 0; k < 8; k++) r |= c[k] << (4 * k);
    o.w[0] = r;
    o.w[1] = 0;
  } else {  // 6 bits, element k at bit 6k
    o.w[0] = c[0] | (c[1] << 6) | (c[2] << 12) | (c[3] << 18) | (c[4] << 24) | (c[5] << 30);
    o.w[1] = (c[5] >> 2) | (c[6] << 4) | (c[7] << 10);
  }
  return o;
}

// INT8 codes of 8 elements (fp32 bits) with scale `code`, round to nearest
// even, for codes at which fp32-subnormal inputs round to zero anyway
// (code >= 8): V / X * 64 = V * 2^(133 - code) is exact, clamped to +-127
// before rounding (the same result as after), and rounded by adding
// 1.5 * 2^23, whose sum's low byte is the two's-complement code.
__device__ __forceinline__ Pack8 int8_convert8(const uint32_t v[8], uint32_t code) {
  const int k = 133 - (int)code;
  uint32_t b[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    float x = __builtin_amdgcn_ldexpf(__builtin_bit_cast(float, v[i]), k);
    x = __builtin_amdgcn_fmed3f(x, -127.0f, 127.0f);
    b[i] = __builtin_bit_cast(uint32_t, x + 12582912.0f);
  }
  Pack8 o;
  // bytes 0 of b[0..3] -> one dword: perm picks byte 0 of each source
  o.w[0] = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u) | __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu);
  o.w[1] = __builtin_amdgcn_perm(b[5], b[4], 0x0C0C0400u) | __builtin_amdgcn_perm(b[7], b[6], 0x04000C0Cu);
  return o;
}

// E2M1 codes of 8 elements with stochastic rounding through gfx950's SR
// conversion.  Measured against the definition on all scale codes 1..254, one
// element per instruction with the seed ~r: where |V / X| >= 1 the discarded
// fraction has at most 22 bits and the instruction rounds up exactly when
// r < F (F: the top 32 bits of that fraction); below 1 it compares only the
// top 22 bits of r and F, so it can differ from the definition only where
// those agree.  It takes fp32-subnormal inputs at their value instead of as
// zero, which matters only for scale codes below 24: from 24 on, a subnormal
// gives |V / X| < 2^-23, whose top 22 fraction bits are zero, and the
// instruction returns the signed zero the flush would give.  The second
// element of a pair takes the seed shifted left by one, so element 2j + 1
// gets its result from the pair (2j, 2j + 1) with the seed ~r >> 1.  `redo`
// is set when an element may differ: bits 16..31 of r equal to bits 6..21 of
// floor(|V / X| * 2^23), a superset of the 22-bit agreement.  Such a group,
// and every block with a scale code below 24, takes the exact conversion.
// Only byte 0 of each result is used: the compiler does not carry the
// instruction's other destination bytes through its first operand.
typedef float v2f __attribute__((ext_vector_type(2)));
template <int J>  // byte J of the packed word: elements 2J (low nibble) and 2J + 1
__device__ __forceinline__ uint32_t sr_fp4_byte(const uint32_t v[8], const uint32_t rnd[8], float S) {
  const v2f pr = {__builtin_bit_cast(float, v[2 * J]), __builtin_bit_cast(float, v[2 * J + 1])};
  const uint32_t lo = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, pr, ~rnd[2 * J], S, 0);
  const uint32_t hi = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, pr, ~rnd[2 * J + 1] >> 1, S, 0);
  return (lo & 0x0Fu) | (hi & ~0x0Fu);  // bits 8..31 unused
}
__device__ __forceinline__ bool sr_fp4_unsure(uint32_t vbits, uint32_t r, int kx) {
  const float f = __builtin_bit_cast(float, vbits);
  const uint32_t key = (uint32_t)__builtin_amdgcn_ldexpf(__builtin_fabsf(f), kx);
  return (key & 0xFFFFu) == (r >> 16);
}
__device__ __forceinline__ uint32_t sr_fp4_hw8(const uint32_t v[8], uint32_t code, const uint32_t rnd[8],
                                               bool& redo) {
  const float S = __builtin_bit_cast(float, code << 23);  // 2^(code - 127), code 24 .. 254
  const int kx = 144 - (int)code;  // |V| * 2^kx = |V / X| * 2^17, below 2^20
  const uint32_t b0 = sr_fp4_byte<0>(v, rnd, S), b1 = sr_fp4_byte<1>(v, rnd, S);
  const uint32_t b2 = sr_fp4_byte<2>(v, rnd, S), b3 = sr_fp4_byte<3>(v, rnd, S);
  bool bad = false;
#pragma unroll
  for (int k = 0; k < 8; k++) bad |= sr_fp4_unsure(v[k], rnd[k], kx);
  redo = bad;
  // byte 0 of b0 .. b3 -> one dword
  return __builtin_amdgcn_perm(b1, b0, 0x0C0C0400u) | __builtin_amdgcn_perm(b3, b2, 0x04000C0Cu);
}

// FP8 (E4M3, E5M2) codes of 8 elements with stochastic rounding through
// gfx950's SR conversion, one element per instruction with the seed ~r.
// Measured against the definition (4M random elements and scale codes, and as
// many again with r agreeing with the discarded fraction in its top 16 to 32
// bits): where the result is normal (|V / X| >= 2^emin) the discarded fraction
// has at most 21 bits and the instruction rounds up exactly when r < F, and it
// saturates like the RNE conversion once fix_sat is applied; where the result
// is subnormal it compares fewer bits than the definition.  So `redo` is set
// for a group holding a nonzero element below 2^emin * X (fp32-subnormal
// inputs included, which the exact conversion flushes), and such a group takes
// the exact conversion.  Needs code + emin >= 1 (the bound is a normal fp32).
template <int F>
__device__ __forceinline__ Pack8 sr_fp8_hw8(const uint32_t v[8], uint32_t code, const uint32_t rnd[8],
                                            bool& redo) {
  const float S = __builtin_bit_cast(float, code << 23);        // 2^(code - 127)
  const uint32_t lim = ((code + Fmt<F>::emin) << 23) - 1u;  // bits of 2^emin * X, less one
  auto cvt = [&](uint32_t old, int k, auto B) {
    constexpr int b = decltype(B)::value;
    const float f = __builtin_bit_cast(float, v[k]);
    if constexpr (F == E4M3) return (uint32_t)__builtin_amdgcn_cvt_scalef32_sr_fp8_f32(old, f, ~rnd[k], S, b);
    else return (uint32_t)__builtin_amdgcn_cvt_scalef32_sr_bf8_f32(old, f, ~rnd[k], S, b);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  using B3 = std::integral_constant<int, 3>;
  Pack8 o;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    uint32_t w = cvt(0u, 4 * h, B0{});
    w = cvt(w, 4 * h + 1, B1{});
    w = cvt(w, 4 * h + 2, B2{});
    w = cvt(w, 4 * h + 3, B3{});
    o.w[h] = fix_sat<F>(w);
  }
  // 2|V| - 2 (the sign shifted out, zeros wrapping to the top), least over
  // the group, against 2 (bound - 1): one shift-add per element, one compare
  uint32_t m = 0xFFFFFFFFu;
#pragma unroll
  for (int k = 0; k < 8; k++) m = umin(m, (v[k] << 1) - 2u);
  redo = m < 2u * lim;
  return o;
}

// Codes of 8 elements of a block with scale `code`.  `v` holds fp32 bits;
// `rnd` the stochastic-rounding words (ignored for RNE).
template <int F, bool SR>
__device__ __forceinline__ Pack8 convert8(const uint32_t v[8], uint32_t code, const uint32_t rnd[8]) {
  if (code == 0xFFu) {  // NaN scale: NaN elements where the format has them
    const uint32_t n = (uint32_t)Fmt<F>::nan;
    uint32_t c[8];
#pragma unroll
    for (int k = 0; k < 8; k++) c[k] = n;
    return pack8<F>(c);
  }
  if (!SR && (F == E4M3 || F == E5M2 || F == E2M1) && code >= (uint32_t)DazFree<F>::value)
    return hw_convert8<F>(v, code);
  if (!SR && F == INT8 && code >= (uint32_t)DazFree<F>::value) return int8_convert8(v, code);
  if (SR && (F == E4M3 || F == E5M2) && code >= (uint32_t)(1 - Fmt<F>::emin)) {  // 0xFF returned above
    bool redo;
    const Pack8 o = sr_fp8_hw8<F>(v, code, rnd, redo);
    if (!redo) return o;
  }
  if (SR && F == E2M1 && code >= 24u) {  // code 0xFF returned above
    bool redo;
    Pack8 o;
    o.w[0] = sr_fp4_hw8(v, code, rnd, redo);
    o.w[1] = 0;
    if (!redo) return o;
  }
  uint32_t c[8];
#pragma unroll
  for (int k = 0; k < 8; k++) c[k] = cvt_exact<F, SR>(v[k], code, SR ? rnd[k] : 0u);
  return pack8<F>(c);
}

}  // namespace mx
