// mx_device.hpp -- device-side building blocks of the MX kernels for gfx950.
//
// Element formats (OCP MX v1.0 / OCP FP8), block conversion steps of
// Algorithm 1 ("Microscaling Data Formats for Deep Learning", summary section 3),
// the Philox4x32-10 generator (Salmon et al., SC'11) used for stochastic
// rounding, and wave-level helpers (DPP).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// ---------------------------------------------------------------------------
// element format traits
// ---------------------------------------------------------------------------
enum { E4M3 = 0, E5M2 = 1, E2M3 = 2, E3M2 = 3, E2M1 = 4, INT8 = 5 };

template <int F> struct Fmt;
// bits: storage bits; mbits: mantissa bits; bias; emin: exponent of the
// smallest normal binade; emax: exponent of the largest normal binade;
// maxcode: code of the largest finite magnitude; nan: code written for a
// block whose scale is NaN.
template <> struct Fmt<E4M3> { static constexpr int bits = 8, mbits = 3, bias = 7,  emin = -6,  emax = 8,  maxcode = 0x7E, nan = 0x7F; };
template <> struct Fmt<E5M2> { static constexpr int bits = 8, mbits = 2, bias = 15, emin = -14, emax = 15, maxcode = 0x7B, nan = 0x7F; };
template <> struct Fmt<E2M3> { static constexpr int bits = 6, mbits = 3, bias = 1,  emin = 0,   emax = 2,  maxcode = 0x1F, nan = 0; };
template <> struct Fmt<E3M2> { static constexpr int bits = 6, mbits = 2, bias = 3,  emin = -2,  emax = 4,  maxcode = 0x1F, nan = 0; };
template <> struct Fmt<E2M1> { static constexpr int bits = 4, mbits = 1, bias = 1,  emin = 0,   emax = 2,  maxcode = 0x7,  nan = 0; };
// INT8: n / 64 with n in [-127, 127]; the scale uses emax = 0.
template <> struct Fmt<INT8> { static constexpr int bits = 8, mbits = 0, bias = 0,  emin = 0,   emax = 0,  maxcode = 127,  nan = 0; };

// Smallest scale code at which every fp32-subnormal input already rounds to
// zero in format F: V < 2^-126 gives |V / X| < 2^(1 - code), below half of the
// smallest grid step.  Blocks at or above it need no explicit flush before a
// hardware conversion.
template <int F> struct DazFree {
  static constexpr int value = (F == INT8) ? 8 : 2 - Fmt<F>::emin + Fmt<F>::mbits;
};

// ---------------------------------------------------------------------------
// scale (Algorithm 1: shared exponent = floor(log2 amax) - emax, E8M0)
// ---------------------------------------------------------------------------
// `amax_bits` is the largest |V| of the block as fp32 bits (sign cleared).
// Inf/NaN anywhere gives a bit pattern >= 0x7F800000 and the NaN scale 0xFF.
// A zero block (and one whose max is fp32-subnormal, which the flush turns
// into a zero block) gets exponent field 0 and so code 0.
template <int F>
__device__ __forceinline__ uint32_t scale_code(uint32_t amax_bits) {
  uint32_t e = amax_bits >> 23;
  if (e >= 255u) return 0xFFu;
  int c = (int)e - Fmt<F>::emax;
  return c < 0 ? 0u : (uint32_t)c;
}

// ---------------------------------------------------------------------------
// exact integer conversion of one element, RNE or SR
// ---------------------------------------------------------------------------
// `vbits`: fp32 bits of a finite V (a subnormal counts as zero, the flush of
// Algorithm 1).  `code`: the block's scale code (not 0xFF).  Computes
// Q(V / 2^(code-127)) on the element grid, the magnitude rounded to nearest
// even (SR == false) or rounded up iff r < floor(frac * 2^32) (SR == true),
// saturating at the largest normal.
//
// With |V| = m * 2^(Ev - 150) and the grid step 2^t of V / X's binade, the
// magnitude in steps is m / 2^sh; one 64-bit shift (m << 32) >> sh leaves n =
// floor(m / 2^sh) in the high word and the top 32 bits of the discarded
// fraction in the low word.  For RNE, sh > 32 means the fraction is below
// 2^-8, so the low word decides ties exactly.
template <int F, bool SR>
__host__ __device__ __forceinline__ uint32_t cvt_exact(uint32_t vbits, uint32_t code, uint32_t r) {
  using T = Fmt<F>;
  const uint32_t sign = vbits >> 31;
  const uint32_t ab = vbits & 0x7FFFFFFFu;
  const int Ev = (int)(ab >> 23);
  const uint32_t m = Ev ? ((ab & 0x7FFFFFu) | 0x800000u) : 0u;
  const int ey = Ev ? Ev - (int)code : -1024;  // exponent of |V / X|; zero: below every grid
  int e = 0, sh;
  if (F == INT8) {
    sh = 17 - ey;  // grid step 2^-6
  } else {
    e = ey < T::emin ? T::emin : ey;
    sh = 23 - T::mbits + (e - ey);
  }
  sh = sh > 63 ? 63 : sh;
  const uint64_t x = ((uint64_t)m << 32) >> sh;
  uint32_t n = (uint32_t)(x >> 32);
  const uint32_t lo = (uint32_t)x;
  if (SR)
    n += r < lo ? 1u : 0u;
  else
    n += (lo > 0x80000000u || (lo == 0x80000000u && (n & 1u))) ? 1u : 0u;
  if (F == INT8) {
    if (n > 127u) n = 127u;
    return sign ? ((0u - n) & 0xFFu) : n;
  }
  // n steps of 2^(e - mbits); for e == emin this covers subnormals and the
  // carry into the first normal binade, and a carry to 2^(mbits+1) moves to the
  // next binade -- all by the same sum.
  uint32_t c = n + ((uint32_t)(e + T::bias - 1) << T::mbits);
  if (c > (uint32_t)T::maxcode) c = T::maxcode;
  return c | (sign << (T::bits - 1));
}

// ---------------------------------------------------------------------------
// flush of fp32-subnormal values to signed zero
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t daz32(uint32_t b) {
  return (b & 0x7F800000u) ? b : (b & 0x80000000u);
}

// ---------------------------------------------------------------------------
// Philox4x32-10
// ---------------------------------------------------------------------------
struct U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ U4 philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                     uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; i++) {
    // one 32 x 32 -> 64-bit multiply gives both halves (V_MAD_U64_U32), and
    // one three-input logic op each new word (truth table 0x96: a ^ b ^ c)
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32(hi1, c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32(hi0, c3, k1, 0x96);
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
  }
  return U4{c0, c1, c2, c3};
}

// The four words for source elements 4g .. 4g+3 (g = i >> 2) of one layout.
__device__ __forceinline__ U4 sr_words(uint64_t seed, uint64_t counter_offset, uint32_t layout,
                                       uint64_t g) {
  const uint64_t j = counter_offset + g;
  return philox((uint32_t)j, (uint32_t)(j >> 32), layout, 0u, (uint32_t)seed,
                (uint32_t)(seed >> 32));
}

// ---------------------------------------------------------------------------
// buffer loads straight into LDS
// ---------------------------------------------------------------------------
typedef int v4i __attribute__((ext_vector_type(4)));

// Raw buffer resource over `bytes` bytes at `p` (gfx9 word 3: 32-bit data),
// in scalar registers.
__device__ __forceinline__ v4i make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// Buffer load of `voff` (+ scalar `soff`) straight into LDS at `lds_dst`
// (wave-uniform; lane i lands at lds_dst + 16 i).  One asm block that also
// sets M0, so the compiler does not model it: every wait on it is explicit,
// and LDS reads of the filled stage come after an asm barrier.  The
// instruction has no register result.  A load that takes its LDS address
// from M0 needs one wait state after the write of M0.
__device__ __forceinline__ void dma16(v4i rs, uint32_t voff, uint32_t soff, uint32_t lds_dst) {
  // a constant offset stays in a scalar register (the instruction takes no
  // literal there)
  asm("" : "+s"(soff));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :
               : "v"(voff), "s"(rs), "s"(lds_dst), "s"(soff)
               : "memory", "m0");
}
// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// ---------------------------------------------------------------------------
// DPP lane exchange inside groups of four lanes
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t quad_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
}
__device__ __forceinline__ uint32_t quad_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
}
__device__ __forceinline__ float quad_xor1f(float v) {
  return __builtin_bit_cast(float, quad_xor1(__builtin_bit_cast(uint32_t, v)));
}
__device__ __forceinline__ float quad_xor2f(float v) {
  return __builtin_bit_cast(float, quad_xor2(__builtin_bit_cast(uint32_t, v)));
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

// fp32 value of 1/sqrt(32) rounded to nearest (0x3E3504F3).
__device__ __forceinline__ float inv_sqrt32() { return __builtin_bit_cast(float, 0x3E3504F3u); }

}  // namespace mx
