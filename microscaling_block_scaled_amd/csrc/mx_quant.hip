// mx_quant.hip -- MX block quantization kernels for gfx950 (CDNA4).
//
// Implements Algorithm 1 of "Microscaling Data Formats for Deep Learning"
// (summary section 3) over 32-element blocks: shared scale from the block max
// (E8M0), per-element conversion with saturation, fp32-subnormal inputs set to
// zero, and the block axis chosen by the output layout.  Optional steps from
// "Format-Aware Fusion for Fast FP4 Pretraining": stochastic rounding with a
// counter-based generator and a fixed-sign 32-point Hadamard transform per
// block before scaling.
//
// Two kernels:
//   k_quant_blocks row-wise layout.  A lane owns one whole 32-element block:
//                  the transform's butterflies and the block max stay in its
//                  registers, and its packed codes go out as one run.
//   k_quant_tiles  column-wise layout stored transposed, optionally fused with
//                  the row-wise one (one HBM read for both).  A 128 x 128 bf16
//                  tile (128 x 64 fp32; 32 KB of LDS) is read with coalesced
//                  16-byte loads, row blocks are emitted from registers with
//                  whole-line streaming stores, the tile is staged in LDS, and
//                  each lane then owns the 32-row column blocks of one dword of
//                  columns (two bf16 or one fp32).  On whole tiles the four
//                  blocks of a column sit in one lane quad, which writes the
//                  column's transposed line in 64-byte runs.
#include "mx_convert.hpp"
#include "mx_device.hpp"
#include "mx_internal.h"

#pragma clang fp contract(off)

namespace mx {

enum { SRC_F32 = 0, SRC_BF16 = 1 };
// ---------------------------------------------------------------------------
// streaming global accesses: every input byte is read once, and the row-wise
// output is written in whole contiguous runs, so these bypass cache residency
// (non-temporal).  The transposed output writes 24-32 byte pieces of many
// rows; those stay ordinary stores so the L2 assembles whole lines.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_stream(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(uint8_t* p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, (u32x4*)p);
}
__device__ __forceinline__ void st_stream(uint8_t* p, uint2 v) {
  __builtin_nontemporal_store(u32x2{v.x, v.y}, (u32x2*)p);
}
__device__ __forceinline__ void st_stream(uint8_t* p, uint32_t v) {
  __builtin_nontemporal_store(v, (uint32_t*)p);
}

// ---------------------------------------------------------------------------
// stores
// ---------------------------------------------------------------------------
// 8 codes at element offset 8 * c of a packed row; non-temporal when NT (a
// writer of whole lines), else ordinary stores that the L2 can merge with the
// neighbouring pieces of the line.
template <int F, bool NT = true>
__device__ __forceinline__ void store8(uint8_t* row, int64_t c, const Pack8& o) {
  if (Fmt<F>::bits == 8) {
    if (NT) st_stream(row + 8 * c, make_uint2(o.w[0], o.w[1]));
    else *(uint2*)(row + 8 * c) = make_uint2(o.w[0], o.w[1]);
  } else if (Fmt<F>::bits == 4) {
    if (NT) st_stream(row + 4 * c, o.w[0]);
    else *(uint32_t*)(row + 4 * c) = o.w[0];
  } else {  // 6 bytes at 6c: dword + half, or half + dword, by parity
    uint8_t* p = row + 6 * c;
    if ((c & 1) == 0) {
      *(uint32_t*)p = o.w[0];
      *(uint16_t*)(p + 4) = (uint16_t)o.w[1];
    } else {
      *(uint16_t*)p = (uint16_t)o.w[0];
      *(uint32_t*)(p + 2) = (o.w[0] >> 16) | (o.w[1] << 16);
    }
  }
}

// 32 codes (a whole block, four Pack8) at an aligned block position (ordinary
// stores: see the streaming note above).
template <int F>
__device__ __forceinline__ void store32(uint8_t* p, const Pack8 o[4]) {
  if (Fmt<F>::bits == 8) {
    *(uint4*)p = make_uint4(o[0].w[0], o[0].w[1], o[1].w[0], o[1].w[1]);
    *(uint4*)(p + 16) = make_uint4(o[2].w[0], o[2].w[1], o[3].w[0], o[3].w[1]);
  } else if (Fmt<F>::bits == 4) {
    *(uint4*)p = make_uint4(o[0].w[0], o[1].w[0], o[2].w[0], o[3].w[0]);
  } else {  // 24 bytes, 8-byte aligned
    const uint32_t w0 = o[0].w[0];
    const uint32_t w1 = (o[0].w[1] & 0xFFFFu) | (o[1].w[0] << 16);
    const uint32_t w2 = (o[1].w[0] >> 16) | (o[1].w[1] << 16);
    const uint32_t w3 = o[2].w[0];
    const uint32_t w4 = (o[2].w[1] & 0xFFFFu) | (o[3].w[0] << 16);
    const uint32_t w5 = (o[3].w[0] >> 16) | (o[3].w[1] << 16);
    *(uint2*)p = make_uint2(w0, w1);
    *(uint2*)(p + 8) = make_uint2(w2, w3);
    *(uint2*)(p + 16) = make_uint2(w4, w5);
  }
}

// ---------------------------------------------------------------------------
// Hadamard-32
// ---------------------------------------------------------------------------
// Block spread over a quad: lane q holds elements 8q .. 8q+7.  Stages with
// stride 1, 2, 4 are inside the lane, 8 and 16 pair lanes q^1 and q^2.  Each
// pair (x_j, x_{j+h}) becomes (x_j + x_{j+h}, x_j - x_{j+h}): the lane holding
// x_{j+h} computes x_j + (-x_{j+h}), the same single rounding.  `sw` are the
// lane's sign masks (bit 31 set where element 8q + k is negated first).
struct HadLane {
  uint32_t sw[8];
  uint32_t flip1, flip2;  // sign bit set on the lanes that subtract in stage 8 / 16
};
__device__ __forceinline__ HadLane had_lane(uint32_t signs, int q) {
  HadLane h;
#pragma unroll
  for (int k = 0; k < 8; k++) h.sw[k] = ((signs >> (8 * q + k)) & 1u) << 31;
  h.flip1 = (uint32_t)(q & 1) << 31;
  h.flip2 = (uint32_t)(q & 2) << 30;
  return h;
}
__device__ __forceinline__ void hadamard_quad(uint32_t v[8], const HadLane& hl) {
  float f[8];
#pragma unroll
  for (int k = 0; k < 8; k++) f[k] = __builtin_bit_cast(float, v[k] ^ hl.sw[k]);
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      if (k & h) continue;
      const float a = f[k], b = f[k + h];
      f[k] = a + b;
      f[k + h] = a - b;
    }
  }
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const float o = quad_xor1f(f[k]);
    f[k] = o + __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f[k]) ^ hl.flip1);
  }
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const float o = quad_xor2f(f[k]);
    f[k] = o + __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f[k]) ^ hl.flip2);
  }
  const float c = inv_sqrt32();
#pragma unroll
  for (int k = 0; k < 8; k++) v[k] = __builtin_bit_cast(uint32_t, f[k] * c);
}

// Whole block in one lane.
__device__ __forceinline__ void hadamard_local(uint32_t v[32], uint32_t signs) {
  if (signs) {  // wave-uniform: the plain Sylvester matrix skips the flips
#pragma unroll
    for (int k = 0; k < 32; k++) v[k] ^= ((signs >> k) & 1u) << 31;
  }
  float f[32];
#pragma unroll
  for (int k = 0; k < 32; k++) f[k] = __builtin_bit_cast(float, v[k]);
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int k = 0; k < 32; k++) {
      if (k & h) continue;
      const float a = f[k], b = f[k + h];
      f[k] = a + b;
      f[k + h] = a - b;
    }
  }
  const float c = inv_sqrt32();
#pragma unroll
  for (int k = 0; k < 32; k++) v[k] = __builtin_bit_cast(uint32_t, f[k] * c);
}

// ---------------------------------------------------------------------------
// shared per-chunk row-wise step
// ---------------------------------------------------------------------------
struct QP {
  const uint8_t* x;
  // rows, cols: the source's extent padded to whole blocks (multiples of 32);
  // they give every pitch, block count and stochastic-rounding index.
  // rows_x, cols_x: the extent that exists in memory; elements past it read
  // as +0 (a short last block is padded with zeros).
  int64_t rows, cols, ld_bytes;
  int64_t rows_x, cols_x;
  uint8_t* q_row;
  int64_t qr_pitch;  // bytes per packed output row (row-wise layout)
  uint8_t* s_row;
  uint8_t* q_colt;
  int64_t qc_pitch;  // bytes per packed output row (transposed layout)
  uint8_t* s_colt;
  uint64_t seed, off;
  uint32_t signs;
  int tiles_r, tiles_c;  // tile kernel: tiles along rows / columns
  int xb;                // tile kernel: side of the square tile blocks run on one XCD (0: none)
  int wpr;               // block kernel: waves per row (64 blocks each)
};

template <int SRC>
__device__ __forceinline__ void widen8(const uint32_t* raw, uint32_t v[8]) {
  if (SRC == SRC_BF16) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = raw[i] << 16;
      v[2 * i + 1] = raw[i] & 0xFFFF0000u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = raw[i];
  }
}

// Quantize the 8 elements v (fp32 bits) at row r, chunk c (elements 8c..8c+7)
// into the row-wise layout.  The four lanes of the block are one DPP quad, q =
// c & 3 is this lane's place in it (the same for every chunk of a lane; `hl`
// holds its Hadamard constants).  All four lanes must be active.  Inputs are
// flushed before the transform; after it no flush is needed: a subnormal
// block maximum gives scale code 0 either way, and the conversions treat a
// subnormal element as zero.
template <int F, bool SR, bool HAD, bool NT = true>
__device__ __forceinline__ void row_chunk(const QP& p, int64_t r, int64_t c, uint32_t v[8],
                                          const HadLane& hl) {
  const int q = (int)(c & 3);
  if (HAD) {
#pragma unroll
    for (int k = 0; k < 8; k++) v[k] = daz32(v[k]);
    hadamard_quad(v, hl);
  }
  uint32_t am = 0;
#pragma unroll
  for (int k = 0; k < 8; k++) am = umax(am, v[k] & 0x7FFFFFFFu);
  am = umax(am, quad_xor1(am));
  am = umax(am, quad_xor2(am));
  const uint32_t code = scale_code<F>(am);
  if (q == 0) p.s_row[r * (p.cols >> 5) + (c >> 2)] = (uint8_t)code;
  uint32_t rnd[8];
  if (SR) {
    const uint64_t g = (uint64_t)(r * p.cols + 8 * c) >> 2;
    const U4 a = sr_words(p.seed, p.off, 0u, g);
    const U4 b = sr_words(p.seed, p.off, 0u, g + 1);
    rnd[0] = a.x; rnd[1] = a.y; rnd[2] = a.z; rnd[3] = a.w;
    rnd[4] = b.x; rnd[5] = b.y; rnd[6] = b.z; rnd[7] = b.w;
  }
  const Pack8 o = convert8<F, SR>(v, code, rnd);
  store8<F, NT>(p.q_row + r * p.qr_pitch, c, o);
}

// row_chunk for 8 bf16 elements held packed in raw[4], without stochastic
// rounding or the transform, for formats with a hardware conversion: the
// block max and the conversion work on the packed pairs.
//  `sc`: where the block's scale byte goes instead of s_row when not null (a
// staging buffer in LDS).
template <int F, bool NT = true>
__device__ __forceinline__ void row_chunk_bf16(const QP& p, int64_t r, int64_t c, const uint32_t raw[4],
                                               uint8_t* sc = nullptr) {
  const int q = (int)(c & 3);
  const uint32_t m = pk_max_u16(pk_max_u16(raw[0] & 0x7FFF7FFFu, raw[1] & 0x7FFF7FFFu),
                                pk_max_u16(raw[2] & 0x7FFF7FFFu, raw[3] & 0x7FFF7FFFu));
  uint32_t am = umax(m << 16, m & 0xFFFF0000u);  // as fp32 bits
  am = umax(am, quad_xor1(am));
  am = umax(am, quad_xor2(am));
  const uint32_t code = scale_code<F>(am);
  if (q == 0) {
    if (sc) *sc = (uint8_t)code;
    else p.s_row[r * (p.cols >> 5) + (c >> 2)] = (uint8_t)code;
  }
  Pack8 o;
  if (hw_ok<F>(code)) {
    o = hw_convert8_bf16<F>(raw, code);
  } else {
    uint32_t v[8], rnd[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = raw[i] << 16;
      v[2 * i + 1] = raw[i] & 0xFFFF0000u;
    }
    o = convert8<F, false>(v, code, rnd);
  }
  store8<F, NT>(p.q_row + r * p.qr_pitch, c, o);
}

// ---------------------------------------------------------------------------
// block kernel: row-wise layout with one whole block per lane
// ---------------------------------------------------------------------------
// All five butterfly stages of the transform run in a lane's registers (no
// lane exchanges), and the block max needs no reduction across lanes.  Wave g
// of the grid takes 64 consecutive blocks of row g / wpr; a lane reads its
// block's 64 (bf16) or 128 (fp32) bytes and writes its packed codes as one run.

// A lane's run of codes: FP4's 16 bytes go out as one streaming store; 8-bit
// and FP6 runs take two or three stores each, whose pieces interleave with the
// neighbouring lanes', so they are ordinary stores that the L2 assembles into
// whole lines.
template <int F>
__device__ __forceinline__ void store32_stream(uint8_t* p, const Pack8 o[4]) {
  if (Fmt<F>::bits == 4) {
    st_stream(p, make_uint4(o[0].w[0], o[1].w[0], o[2].w[0], o[3].w[0]));
  } else {
    store32<F>(p, o);
  }
}

// `n` elements (8 or 32) of ESZ bytes at src into raw words (two bf16 or one
// fp32 per word), of which the first `valid` exist and the rest read +0: whole
// 16-byte loads when all exist, else element by element (only the short last
// block of a row or tile).
template <int ESZ, int n, bool NT>
__device__ __forceinline__ void load_elems(const uint8_t* src, int valid, uint32_t* raw) {
  constexpr int W = n * ESZ / 4;  // words
  if (valid >= n) {
#pragma unroll
    for (int j = 0; j < W / 4; j++) {
      const uint4 t = NT ? ld_stream(src + 16 * j) : *(const uint4*)(src + 16 * j);
      raw[4 * j] = t.x; raw[4 * j + 1] = t.y; raw[4 * j + 2] = t.z; raw[4 * j + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int w = 0; w < W; w++) {
      if (ESZ == 4) {
        raw[w] = w < valid ? *(const uint32_t*)(src + 4 * w) : 0u;
      } else {
        const uint32_t lo = 2 * w < valid ? *(const uint16_t*)(src + 4 * w) : 0u;
        const uint32_t hi = 2 * w + 1 < valid ? *(const uint16_t*)(src + 4 * w + 2) : 0u;
        raw[w] = lo | (hi << 16);
      }
    }
  }
}

template <int SRC, int F, bool SR, bool HAD>
__global__ __launch_bounds__(256) void k_quant_blocks(QP p) {
  constexpr int ESZ = SRC == SRC_BF16 ? 2 : 4;
  // bf16 without SR or the transform, formats with a hardware conversion: the
  // packed-pair path (block max and conversion on bf16 pairs)
  constexpr bool PACKED = SRC == SRC_BF16 && !HAD && HwPath32<F, SR>::value;
  const int lane = threadIdx.x & 63;
  // wave-uniform 32-bit index arithmetic (the host keeps rows * wpr < 2^32)
  const uint32_t g = blockIdx.x * 4u + (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t wpr = (uint32_t)p.wpr;
  const int64_t r = g / wpr;
  const int64_t kb = (int64_t)(g % wpr) * 64 + lane;  // block of row r
  const int64_t bpr = p.cols >> 5;
  if (r >= p.rows_x || kb >= bpr) return;  // no lane exchanges below
  const uint8_t* src = p.x + r * p.ld_bytes + kb * 32 * ESZ;
  uint32_t raw[8 * ESZ];
  load_elems<ESZ, 32, false>(src, (int)(p.cols_x - kb * 32 < 32 ? p.cols_x - kb * 32 : 32), raw);
  uint32_t v[32];
  uint32_t am = 0;
  if constexpr (PACKED) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) m = pk_max_u16(m, raw[i] & 0x7FFF7FFFu);
    am = umax(m << 16, m & 0xFFFF0000u);
  } else {
    // Flush subnormal inputs before the transform.  For bf16 a block is first
    // checked on the packed pairs: per half, 2 h - 2 (mod 2^16) drops the sign
    // bit, wraps zero to 0xFFFE and lands below 0xFD only for a subnormal (one
    // packed multiply-add); only lanes holding one flush.
    bool sub = true;
    if constexpr (SRC == SRC_BF16 && HAD) {
      u16x2 mn = {0xFFFF, 0xFFFF};
#pragma unroll
      for (int i = 0; i < 16; i++) {
        uint32_t t;  // per half: h * 2 + 0xFFFE (the compiler would split it in two)
        asm("v_pk_mad_u16 %0, %1, 2, -2" : "=v"(t) : "v"(raw[i]));
        mn = __builtin_elementwise_min(mn, __builtin_bit_cast(u16x2, t));
      }
      sub = mn.x < 0xFD || mn.y < 0xFD;
    }
#pragma unroll
    for (int j = 0; j < 4; j++) widen8<SRC>(&raw[j * 2 * ESZ], &v[8 * j]);
    if (HAD) {
      if (sub) {
#pragma unroll
        for (int k = 0; k < 32; k++) v[k] = daz32(v[k]);
      }
      hadamard_local(v, p.signs);
    }
#pragma unroll
    for (int k = 0; k < 32; k++) am = umax(am, v[k] & 0x7FFFFFFFu);
  }
  const uint32_t code = scale_code<F>(am);
  p.s_row[r * bpr + kb] = (uint8_t)code;
  Pack8 o[4];
  bool fast = false;
  if constexpr (PACKED && (F == E2M3 || F == E3M2)) {
    if (hw_ok<F>(code)) {
      hw_convert32_bf16_fp6<F>(raw, code, o);
      fast = true;
    }
  } else if constexpr (HwPath<F, SR>::value) {
    if (hw_ok<F>(code)) {
#pragma unroll
      for (int h = 0; h < 4; h++) {
        if constexpr (PACKED)
          o[h] = hw_convert8_bf16<F>(&raw[4 * h], code);
        else
          o[h] = hw_convert8<F>(&v[8 * h], code);
      }
      fast = true;
    }
  }
  if (!fast) {
    if constexpr (PACKED) {
#pragma unroll
      for (int j = 0; j < 4; j++) widen8<SRC>(&raw[j * 2 * ESZ], &v[8 * j]);
    }
#pragma unroll
    for (int h = 0; h < 4; h++) {
      uint32_t rnd[8];
      if (SR) {
        const uint64_t c = (uint64_t)(r * p.cols + kb * 32 + 8 * h) >> 2;
        const U4 a = sr_words(p.seed, p.off, 0u, c);
        const U4 b = sr_words(p.seed, p.off, 0u, c + 1);
        rnd[0] = a.x; rnd[1] = a.y; rnd[2] = a.z; rnd[3] = a.w;
        rnd[4] = b.x; rnd[5] = b.y; rnd[6] = b.z; rnd[7] = b.w;
      }
      o[h] = convert8<F, SR>(&v[8 * h], code, rnd);
    }
  }
  store32_stream<F>(p.q_row + r * p.qr_pitch + kb * 4 * Fmt<F>::bits, o);
}

// ---------------------------------------------------------------------------
// tile kernel: transposed column-wise layout, optionally fused with row-wise
// ---------------------------------------------------------------------------
template <int SRC> struct TileShape {
  static constexpr int ESZ = SRC == SRC_BF16 ? 2 : 4;  // source bytes per element
  static constexpr int TC = 256 / ESZ;         // tile columns: 256 bytes of a source row
  static constexpr int TR = 128;               // tile rows: four column blocks
  static constexpr int ROWB = 256;             // LDS bytes per tile row
  static constexpr int CPRW = TC / 8;          // 8-element chunks per tile row
  static constexpr int RPP = 256 / CPRW;       // tile rows per load pass
  static constexpr int PASSES = TR / RPP;
  static constexpr int RAWN = SRC == SRC_BF16 ? 4 : 8;  // dwords per chunk
  static constexpr int CPT = TC / 64;          // columns per lane, column pass
};

// Scale code and packed codes of the column block at column `col`, rows
// rs .. rs + 31 (v: its 32 elements as fp32 bits).
template <int F, bool SR, bool HAD>
__device__ __forceinline__ uint32_t col_codes(const QP& p, uint32_t v[32], int64_t col, int64_t rs,
                                              Pack8 o[4]) {
  if (HAD) {
#pragma unroll
    for (int k = 0; k < 32; k++) v[k] = daz32(v[k]);
    hadamard_local(v, p.signs);
  }
  uint32_t am = 0;
#pragma unroll
  for (int k = 0; k < 32; k++) am = umax(am, v[k] & 0x7FFFFFFFu);
  const uint32_t code = scale_code<F>(am);
#pragma unroll
  for (int h = 0; h < 4; h++) {
    uint32_t rnd[8];
    if (SR) {
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const uint64_t i = (uint64_t)((rs + 8 * h + k) * p.cols + col);
        const U4 w = sr_words(p.seed, p.off, 1u, i >> 2);
        const uint32_t s = (uint32_t)(i & 3);
        rnd[k] = s == 0 ? w.x : (s == 1 ? w.y : (s == 2 ? w.z : w.w));
      }
    }
    o[h] = convert8<F, SR>(&v[8 * h], code, rnd);
  }
  return code;
}

template <int F, bool SR, bool HAD>
__device__ __forceinline__ void col_block(const QP& p, uint32_t v[32], int64_t col, int64_t rs) {
  Pack8 o[4];
  const uint32_t code = col_codes<F, SR, HAD>(p, v, col, rs, o);
  p.s_colt[col * (p.rows >> 5) + (rs >> 5)] = (uint8_t)code;
  store32<F>(p.q_colt + col * p.qc_pitch + (rs * Fmt<F>::bits) / 8, o);
}

template <int CTRL>
__device__ __forceinline__ uint32_t quad_perm(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// Column block qb (rows r0 + 32 qb ..) of column `col`, held by lane qb of a
// quad whose four lanes hold the column's four blocks of the tile.  With
// 8-bit codes the quad's 128 transposed bytes are exchanged so that each store
// instruction writes 64 contiguous bytes per quad: lane q first writes bytes
// 16 q .. 16 q + 15 (half q & 1 of block q >> 1), then 64 + 16 q .. (half
// q & 1 of block 2 + (q >> 1)).
template <int F, bool SCALE = true>
__device__ __forceinline__ void col_quad_store(const QP& p, const Pack8 o[4], uint32_t code, int64_t col,
                                               int64_t r0, int qb) {
  const int64_t rs = r0 + 32 * qb;
  if (SCALE) p.s_colt[col * (p.rows >> 5) + (rs >> 5)] = (uint8_t)code;
  if (Fmt<F>::bits == 8) {
    const uint32_t d[8] = {o[0].w[0], o[0].w[1], o[1].w[0], o[1].w[1],
                           o[2].w[0], o[2].w[1], o[3].w[0], o[3].w[1]};
    const bool odd = qb & 1;
    uint32_t e[8];
#pragma unroll
    for (int m = 0; m < 4; m++) {
      // Both halves are moved on every lane before the per-lane choice: the
      // empty asm pins the exchanges to uniform control flow, so the compiler
      // cannot turn the choice into branches that leave source lanes inactive.
      uint32_t a0 = quad_perm<0x50>(d[m]), a1 = quad_perm<0x50>(d[4 + m]);  // from lanes [0,0,1,1]
      uint32_t b0 = quad_perm<0xFA>(d[m]), b1 = quad_perm<0xFA>(d[4 + m]);  // from lanes [2,2,3,3]
      asm volatile("" : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1));
      e[m] = odd ? a1 : a0;
      e[4 + m] = odd ? b1 : b0;
    }
    uint8_t* line = p.q_colt + col * p.qc_pitch + r0;
    *(uint4*)(line + 16 * qb) = make_uint4(e[0], e[1], e[2], e[3]);
    *(uint4*)(line + 64 + 16 * qb) = make_uint4(e[4], e[5], e[6], e[7]);
  } else {
    store32<F>(p.q_colt + col * p.qc_pitch + (rs * Fmt<F>::bits) / 8, o);
  }
}

template <int F, bool SR, bool HAD>
__device__ __forceinline__ void col_quad(const QP& p, uint32_t v[32], int64_t col, int64_t r0, int qb) {
  Pack8 o[4];
  const uint32_t code = col_codes<F, SR, HAD>(p, v, col, r0 + 32 * qb, o);
  col_quad_store<F>(p, o, code, col, r0, qb);
}

// Column pass on bf16 pairs with stochastic rounding: w[i] holds columns col
// (low half, col even) and col + 1 (high half) of row rs + i.  One Philox call
// gives the words of a row's group of four columns (element index i = row *
// cols + col with cols % 4 == 0), so one call serves both columns.  In whole
// tiles (WHOLE, rs = r0 + 32 qb) the lane ^ 4 holds the group's other pair
// for the same rows: per 8-row chunk each lane of the pair makes the calls of
// four rows and hands the other its two words of each (a quarter of the calls
// of one call per element; needs every lane of the wave active), and the
// codes go out through the quad exchange.  Ragged tiles make all of a chunk's
// calls themselves and store plainly.  Both columns' scale codes come first;
// the chunks then convert both columns, so only one chunk's words are live.
template <int F, bool HAD, bool WHOLE>
__device__ __forceinline__ void col_pair_sr(const QP& p, const uint32_t w[32], int64_t col, int64_t r0,
                                            int qb) {
  const int64_t rs = r0 + 32 * qb;
  uint32_t v[2][32];
#pragma unroll
  for (int i = 0; i < 32; i++) {
    v[0][i] = w[i] << 16;
    v[1][i] = w[i] & 0xFFFF0000u;
  }
  uint32_t code[2];
#pragma unroll
  for (int k = 0; k < 2; k++) {
    if (HAD) {
#pragma unroll
      for (int i = 0; i < 32; i++) v[k][i] = daz32(v[k][i]);
      hadamard_local(v[k], p.signs);
    }
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 32; i++) am = umax(am, v[k][i] & 0x7FFFFFFFu);
    code[k] = scale_code<F>(am);
  }
  const bool hi = (col >> 1) & 1;  // second pair of its group of four
  const int64_t g0 = col & ~(int64_t)3;
  Pack8 o[2][4];
#pragma unroll
  for (int h = 0; h < 4; h++) {
    uint32_t rnd[2][8];
    if constexpr (!WHOLE) {
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const U4 wd = sr_words(p.seed, p.off, 1u, (uint64_t)((rs + 8 * h + j) * p.cols + g0) >> 2);
        rnd[0][j] = hi ? wd.z : wd.x;
        rnd[1][j] = hi ? wd.w : wd.y;
      }
    } else {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      // this lane's calls: chunk rows 4 hi + j; the partner's: 4 (1 - hi) + j
      const int64_t row = rs + 8 * h + (hi ? 4 : 0) + j;
      const U4 wd = sr_words(p.seed, p.off, 1u, (uint64_t)(row * p.cols + g0) >> 2);
      const uint32_t own0 = hi ? wd.z : wd.x, own1 = hi ? wd.w : wd.y;
      uint32_t oth0 = hi ? wd.x : wd.z, oth1 = hi ? wd.y : wd.w;
      asm volatile("" : "+v"(oth0), "+v"(oth1));
      // bit-mask swizzle: lane ^ 4 within each group of 32
      const uint32_t in0 = (uint32_t)__builtin_amdgcn_ds_swizzle((int)oth0, 0x101F);
      const uint32_t in1 = (uint32_t)__builtin_amdgcn_ds_swizzle((int)oth1, 0x101F);
      rnd[0][j] = hi ? in0 : own0;
      rnd[1][j] = hi ? in1 : own1;
      rnd[0][4 + j] = hi ? own0 : in0;
      rnd[1][4 + j] = hi ? own1 : in1;
    }
    }
#pragma unroll
    for (int k = 0; k < 2; k++) o[k][h] = convert8<F, true>(&v[k][8 * h], code[k], rnd[k]);
  }
  if constexpr (WHOLE) {
    col_quad_store<F>(p, o[0], code[0], col, r0, qb);
    col_quad_store<F>(p, o[1], code[1], col + 1, r0, qb);
  } else {
#pragma unroll
    for (int k = 0; k < 2; k++) {
      if (col + k >= p.cols_x) break;  // a column past the source's end
      p.s_colt[(col + k) * (p.rows >> 5) + (rs >> 5)] = (uint8_t)code[k];
      store32<F>(p.q_colt + (col + k) * p.qc_pitch + (rs * Fmt<F>::bits) / 8, o[k]);
    }
  }
}

// Whole-tile column pass on bf16 pairs without stochastic rounding or the
// transform, for formats with a hardware conversion: w[i] holds columns col
// (low half) and col + 1 (high half) of row 32 qb + i.  Both block maxima come
// from one packed max; each column's pairs of rows are regrouped with a byte
// permute for the packed conversion.
template <int F>
__device__ __forceinline__ void col_pair_bf16(const QP& p, const uint32_t w[32], int64_t col, int64_t r0,
                                              int qb) {
  const bool gather = (p.rows & 127) == 0;  // a quad's scale bytes make an aligned dword
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 32; i++) m = pk_max_u16(m, w[i] & 0x7FFF7FFFu);
  const uint32_t codes[2] = {scale_code<F>(m << 16), scale_code<F>(m & 0xFFFF0000u)};
  // The quad's four scale bytes of each column are one dword of s_colt: lane
  // 0 of the quad writes the first column's, lane 1 the second's.
  uint32_t g[2];
#pragma unroll
  for (int k = 0; k < 2; k++) {
    uint32_t a = quad_perm<0xB1>(codes[k]);  // from lanes [1,0,3,2]
    asm volatile("" : "+v"(a));
    a = codes[k] | (a << 8);
    uint32_t b = quad_perm<0x4E>(a);  // from lanes [2,3,0,1]
    asm volatile("" : "+v"(b));
    g[k] = a | (b << 16);  // complete on lane 0
  }
  uint32_t g1 = quad_perm<0x00>(g[1]);  // lane 0's to every lane
  asm volatile("" : "+v"(g1));
  if (gather && qb < 2)
    *(uint32_t*)(p.s_colt + (col + qb) * (p.rows >> 5) + (r0 >> 5)) = qb == 0 ? g[0] : g1;
#pragma unroll
  for (int k = 0; k < 2; k++) {
    const uint32_t code = codes[k];
    Pack8 o[4];
    if (hw_ok<F>(code)) {
      uint32_t pr[16];  // rows 2 j, 2 j + 1 of this column
#pragma unroll
      for (int j = 0; j < 16; j++)
        pr[j] = __builtin_amdgcn_perm(w[2 * j + 1], w[2 * j], k == 0 ? 0x05040100u : 0x07060302u);
      if constexpr (F == E2M3 || F == E3M2) {
        hw_convert32_bf16_fp6<F>(pr, code, o);
      } else {
#pragma unroll
        for (int h = 0; h < 4; h++) o[h] = hw_convert8_bf16<F>(&pr[4 * h], code);
      }
    } else {
      uint32_t v[32], rnd[8];
#pragma unroll
      for (int i = 0; i < 32; i++) v[i] = k == 0 ? w[i] << 16 : w[i] & 0xFFFF0000u;
#pragma unroll
      for (int h = 0; h < 4; h++) o[h] = convert8<F, false>(&v[8 * h], code, rnd);
    }
    if (!gather) p.s_colt[(col + k) * (p.rows >> 5) + (r0 >> 5) + qb] = (uint8_t)code;
    col_quad_store<F, false>(p, o, code, col + k, r0, qb);
  }
}

// 16-byte piece p of tile row r sits at piece p ^ tile_swz(r) of its LDS row
// in a whole tile: the column pass reads rows 32 apart together, and rows 32
// apart fall in different banks.
__device__ __forceinline__ int tile_swz(int r) { return ((r >> 5) & 3) * 4; }

// Whole tiles: the column pass gives lane 4 c + qb of wave w the dword
// 16 w + c of rows 32 qb .. 32 qb + 31, so a quad holds the four blocks of its
// columns (one 128-byte transposed line each for 8-bit codes).  Ragged edge
// tiles: wave qb takes rows 32 qb .., lane g the dword g.
template <int SRC, int F, bool SR, bool HAD, bool ROWS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SR && SRC == SRC_BF16 ? 3 : 1))) void k_quant_tiles(QP p) {
  using T = TileShape<SRC>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[T::TR * T::ROWB];
  __shared__ uint32_t sc_lds[T::TR];  // row-wise scale bytes of a whole tile, one dword per row
  const int tid = threadIdx.x;
  // Workgroups reach the 8 XCDs round-robin.  With xb > 0 the tiles go out in
  // xb x xb blocks, each block on one XCD (its workgroups 8 apart): the xb
  // tiles that write one 32-byte sector of a row's scales (or of a column's
  // transposed scales) then write it through one L2, which merges their
  // 4-byte pieces into whole sectors.  Blocks are interleaved over the XCDs,
  // so the tiles running together still cover a compact band of the tensor.
  int64_t tr, tc;
  if (p.xb) {
    const int64_t b = blockIdx.x, x = b % 8, l = b / 8, S = (int64_t)p.xb * p.xb;
    const int64_t blk = (l / S) * 8 + x, i = l % S, kb = p.tiles_c / p.xb;
    tr = p.xb * (blk / kb) + i / p.xb;
    tc = p.xb * (blk % kb) + i % p.xb;
  } else {
    tr = blockIdx.x / p.tiles_c;
    tc = blockIdx.x % p.tiles_c;
  }
  const int64_t r0 = tr * T::TR, c0 = tc * T::TC;
  // rows / columns of the tile that exist, and the same padded to whole
  // blocks (the padding reads +0)
  const int tr_eff = (int)(p.rows_x - r0 < T::TR ? p.rows_x - r0 : T::TR);
  const int tc_eff = (int)(p.cols_x - c0 < T::TC ? p.cols_x - c0 : T::TC);
  const int tr_pad = (int)(p.rows - r0 < T::TR ? p.rows - r0 : T::TR);
  const int tc_pad = (int)(p.cols - c0 < T::TC ? p.cols - c0 : T::TC);
  const bool whole_tile = tr_eff == T::TR && tc_eff == T::TC;
  // whole bf16 tiles with rows of s_row in whole dwords: the row-wise scales
  // are gathered in LDS and written one dword per row
  constexpr bool FAST = SRC == SRC_BF16 && !HAD && HwPath<F, SR>::value;
  constexpr bool FASTCOL = SRC == SRC_BF16 && !HAD && HwPath32<F, SR>::value;
  // The tile's work, compiled twice: for whole tiles (WH: straight-line
  // 16-byte loads, so the compiler counts them exactly and the first passes
  // can start before the last loads land) and for ragged ones.
  auto body = [&](auto WH_) {
    constexpr bool WH = decltype(WH_)::value;
    constexpr bool whole = WH;
    const bool gather = FAST && ROWS && whole && (p.cols & 127) == 0;
    const int cq = tid % T::CPRW, sub = tid / T::CPRW;
    const HadLane hl = had_lane(p.signs, cq & 3);  // tile columns start at a multiple of 4 chunks
    // chunk cq (8 elements) takes part when it lies in a block of the padded
    // tile; `valid` of its elements exist
    const bool col_ok = cq * 8 < tc_pad;
    const int valid = tc_eff - cq * 8;

    uint32_t raw[T::PASSES][T::RAWN];
    if constexpr (WH) {
      // every chunk exists: whole 16-byte loads, in pass order
#pragma unroll
      for (int pp = 0; pp < T::PASSES; pp++) {
        const uint8_t* src = p.x + (r0 + pp * T::RPP + sub) * p.ld_bytes + (c0 + 8 * cq) * T::ESZ;
#pragma unroll
        for (int j = 0; j < T::RAWN / 4; j++) {
          const uint4 t = ld_stream(src + 16 * j);
          raw[pp][4 * j] = t.x; raw[pp][4 * j + 1] = t.y; raw[pp][4 * j + 2] = t.z; raw[pp][4 * j + 3] = t.w;
        }
      }
      // the first half of the passes goes ahead while the second half's
      // loads are in flight
      __builtin_amdgcn_s_waitcnt(0x0F70 | (T::RAWN / 4) * (T::PASSES / 2));
    } else {
#pragma unroll
      for (int pp = 0; pp < T::PASSES; pp++) {
        const int row = pp * T::RPP + sub;
        if (row < tr_pad && col_ok) {
          if (row < tr_eff && valid > 0) {
            const uint8_t* src = p.x + (r0 + row) * p.ld_bytes + (c0 + 8 * cq) * T::ESZ;
            load_elems<T::ESZ, 8, true>(src, valid, raw[pp]);
          } else {
#pragma unroll
            for (int k = 0; k < T::RAWN; k++) raw[pp][k] = 0u;
          }
        }
      }
      // All of the tile is needed before the first stores go out.  Waiting for
      // the loads here, explicitly, tells the compiler they are complete, so it
      // does not wait again (for the stores then in flight) before each pass.
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
#pragma unroll
    for (int pp = 0; pp < T::PASSES; pp++) {
      const int row = pp * T::RPP + sub;
      if (WH || (row < tr_pad && col_ok)) {
        uint32_t v[8];
        widen8<SRC>(raw[pp], v);
        if (ROWS && (WH || row < tr_eff)) {
          if constexpr (FAST) {
            row_chunk_bf16<F>(p, r0 + row, (c0 >> 3) + cq, raw[pp],
                              gather ? (uint8_t*)sc_lds + 4 * row + (cq >> 2) : nullptr);
          } else {
            uint32_t w[8];
#pragma unroll
            for (int k = 0; k < 8; k++) w[k] = v[k];
            row_chunk<F, SR, HAD>(p, r0 + row, (c0 >> 3) + cq, w, hl);
          }
        }
        const int sw = whole ? tile_swz(row) : 0;
        uint8_t* dst = lds + row * T::ROWB;
        if constexpr (SRC == SRC_BF16) {
          *(uint4*)(dst + 16 * (cq ^ sw)) = make_uint4(raw[pp][0], raw[pp][1], raw[pp][2], raw[pp][3]);
        } else {
          *(uint4*)(dst + 16 * ((2 * cq) ^ sw)) = make_uint4(v[0], v[1], v[2], v[3]);
          *(uint4*)(dst + 16 * ((2 * cq + 1) ^ sw)) = make_uint4(v[4], v[5], v[6], v[7]);
        }
      }
    }
    __syncthreads();

    if (gather && tid < T::TR)
      *(uint32_t*)(p.s_row + (r0 + tid) * (p.cols >> 5) + (c0 >> 5)) = sc_lds[tid];
    if (whole) {
      const int lane = tid & 63, qb = lane & 3;
      const int d = 16 * (tid >> 6) + (lane >> 2);
      const uint8_t* src = lds + 32 * qb * T::ROWB + 16 * ((d >> 2) ^ (4 * qb)) + 4 * (d & 3);
      uint32_t w[32];
#pragma unroll
      for (int i = 0; i < 32; i++) w[i] = *(const uint32_t*)(src + i * T::ROWB);
      if constexpr (FASTCOL) {
        col_pair_bf16<F>(p, w, c0 + 2 * d, r0, qb);
      } else if constexpr (SR && SRC == SRC_BF16) {
        col_pair_sr<F, HAD, true>(p, w, c0 + 2 * d, r0, qb);
      } else {
#pragma unroll
        for (int k = 0; k < T::CPT; k++) {
          uint32_t v[32];
#pragma unroll
          for (int i = 0; i < 32; i++)
            v[i] = SRC == SRC_BF16 ? (k == 0 ? w[i] << 16 : w[i] & 0xFFFF0000u) : w[i];
          col_quad<F, SR, HAD>(p, v, c0 + T::CPT * d + k, r0, qb);
        }
      }
    } else {
      const int qb = tid >> 6, g = tid & 63;
      if (32 * qb < tr_eff && g * T::CPT < tc_eff) {
        uint32_t w[32];
#pragma unroll
        for (int i = 0; i < 32; i++) w[i] = *(const uint32_t*)(lds + (32 * qb + i) * T::ROWB + g * 4);
        if constexpr (SR && SRC == SRC_BF16) {
          col_pair_sr<F, HAD, false>(p, w, c0 + 2 * g, r0, qb);
        } else {
#pragma unroll
          for (int k = 0; k < T::CPT; k++) {
            uint32_t v[32];
#pragma unroll
            for (int i = 0; i < 32; i++)
              v[i] = SRC == SRC_BF16 ? (k == 0 ? w[i] << 16 : w[i] & 0xFFFF0000u) : w[i];
            if (c0 + g * T::CPT + k < p.cols_x) col_block<F, SR, HAD>(p, v, c0 + g * T::CPT + k, r0 + 32 * qb);
          }
        }
      }
    }
  };
  if (whole_tile) body(std::true_type{});
  else body(std::false_type{});
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static QP make_qp(const QuantArgs& a) {
  QP p{};
  p.x = (const uint8_t*)a.x;
  p.rows_x = a.rows;
  p.cols_x = a.cols;
  p.rows = (a.rows + 31) / 32 * 32;
  p.cols = (a.cols + 31) / 32 * 32;
  p.ld_bytes = a.ld_bytes;
  const int bits = elem_bits(a.fmt);
  p.q_row = a.q_row;
  p.qr_pitch = p.cols * bits / 8;
  p.s_row = a.s_row;
  p.q_colt = a.q_colt;
  p.qc_pitch = p.rows * bits / 8;
  p.s_colt = a.s_colt;
  p.seed = a.seed;
  p.off = a.counter_offset;
  p.signs = a.signs;
  return p;
}

template <int SRC, int F, bool SR, bool HAD>
static hipError_t rows_launch(const QP& p0, hipStream_t st) {
  QP p = p0;
  const int64_t wpr = (p.cols / 32 + 63) / 64;  // waves per row, 64 blocks each
  p.wpr = (int)wpr;
  const int64_t waves = p.rows_x * wpr;
  if (waves >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_quant_blocks<SRC, F, SR, HAD>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int SRC, int F, bool SR, bool HAD>
static hipError_t tiles_launch(const QP& p0, bool rows, hipStream_t st) {
  using T = TileShape<SRC>;
  QP p = p0;
  const int64_t tiles_r = (p.rows + T::TR - 1) / T::TR;
  const int64_t tiles_c = (p.cols + T::TC - 1) / T::TC;
  p.tiles_r = (int)tiles_r;
  p.tiles_c = (int)tiles_c;
  const int64_t grid = tiles_r * tiles_c;
  // Fused row + column output: 8 x 8 tile blocks per XCD where the tile grid
  // splits into a multiple of 8 of them.  Each row-wise scale sector then
  // leaves one L2 whole (with round-robin tiles the 32 tiles of a row's scale
  // line ran on all 8 XCDs, and the dual-layout E4M3 kernel on bf16
  // 16384 x 4096 wrote 153.5 MB for 138.4 MB of output; 138.5 MB with the
  // blocks, and 2.7 % faster).  The column-only kernel keeps the round-robin
  // order: its transposed scale sectors are written by tiles 8 apart in one
  // column, which already share an XCD, and the blocks made it slower.
  constexpr int XB = 8;
  p.xb = rows && tiles_r % XB == 0 && tiles_c % XB == 0 && grid % (8 * XB * XB) == 0 ? XB : 0;
  if (rows)
    hipLaunchKernelGGL((k_quant_tiles<SRC, F, SR, HAD, true>), dim3((unsigned)grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((k_quant_tiles<SRC, F, SR, HAD, false>), dim3((unsigned)grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

// Dispatch over (source, format, rounding, Hadamard) to a templated launcher.
template <template <int, int, bool, bool> class L, typename... A>
static hipError_t dispatch(int src, int fmt, bool sr, bool had, A... args) {
#define MX_DISPATCH_F(S, FM)                                                     \
  if (!sr && !had) return L<S, FM, false, false>::run(args...);                  \
  if (!sr && had) return L<S, FM, false, true>::run(args...);                    \
  if (sr && !had) return L<S, FM, true, false>::run(args...);                    \
  return L<S, FM, true, true>::run(args...);
#define MX_DISPATCH_S(S)                    \
  switch (fmt) {                            \
    case E4M3: { MX_DISPATCH_F(S, E4M3) }   \
    case E5M2: { MX_DISPATCH_F(S, E5M2) }   \
    case E2M3: { MX_DISPATCH_F(S, E2M3) }   \
    case E3M2: { MX_DISPATCH_F(S, E3M2) }   \
    case E2M1: { MX_DISPATCH_F(S, E2M1) }   \
    default: { MX_DISPATCH_F(S, INT8) }     \
  }
  if (src == SRC_BF16) { MX_DISPATCH_S(SRC_BF16) }
  MX_DISPATCH_S(SRC_F32)
#undef MX_DISPATCH_S
#undef MX_DISPATCH_F
}

template <int SRC, int F, bool SR, bool HAD> struct RowsL {
  static hipError_t run(const QP& p, hipStream_t st) { return rows_launch<SRC, F, SR, HAD>(p, st); }
};
template <int SRC, int F, bool SR, bool HAD> struct TilesL {
  static hipError_t run(const QP& p, bool rows, hipStream_t st) {
    return tiles_launch<SRC, F, SR, HAD>(p, rows, st);
  }
};

hipError_t launch_quant_rows(const QuantArgs& a, hipStream_t st) {
  const QP p = make_qp(a);
  return dispatch<RowsL>(a.src, a.fmt, a.round == 1, a.hadamard, p, st);
}

hipError_t launch_quant_tiles(const QuantArgs& a, bool with_rows, hipStream_t st) {
  const QP p = make_qp(a);
  return dispatch<TilesL>(a.src, a.fmt, a.round == 1, a.hadamard, p, with_rows, st);
}

}  // namespace mx
