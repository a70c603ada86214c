// mx_gemm_kernels.hpp -- block-scaled MX matrix multiply on gfx950's
// V_MFMA_SCALE_F32_{16X16X128,32X32X64}_F8F6F4 (kernel templates; the build
// compiles one unit per operand-format pair that instantiates gemm_launch,
// and mx_gemm.hip dispatches to them).
//
// C[m,n] = sum over 32-element blocks kb of 2^(sa[m,kb]-127) * 2^(sb[n,kb]-127)
//          * sum_{k in kb} P_A[m,k] * P_B[n,k]
// ("Microscaling Data Formats for Deep Learning", summary section 4: dot
// products consume MX operands and return scalar floats; section 2: v = X * P).
// The E8M0 scales are applied inside the matrix instruction, accumulation is
// fp32 and C is fp32 (or bf16, or MX).
//
// General kernel (k_gemm; any K % 32 == 0): a 256-thread workgroup computes a
// 256 x 256 tile of C; its four waves each own 128 x 128 (8 x 8 instructions
// of 16 x 16 x 128).  Per K-step of 128 elements the A and B panels (256 rows
// each, with their scale bytes) are copied global -> registers -> LDS, double
// buffered, so the copy of step s+1 overlaps the instructions of step s.
//
// Operand lane layouts of the 16x16x128 instruction (lane l, row l % 16, block
// kb = l / 16 of the K-step; the scale operand of lane l is the E8M0 byte of
// that row and block):
//   FP8 (E4M3, E5M2): 32 bytes = K-step bytes [16 kb, 16 kb + 16) followed by
//                     [64 + 16 kb, 64 + 16 kb + 16)
//   FP6 (E2M3, E3M2): the 24 packed bytes of block kb
//   FP4 (E2M1):       the 16 packed bytes of block kb
// Result: lane l holds C rows 4 (l / 16) + v, v = 0..3, column l % 16.
#pragma once

#include <atomic>
#include <utility>

#include "mx_convert.hpp"
#include "mx_device.hpp"
#include "mx_internal.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int BM = 256, BN = 256, KS = 128;

template <int F> struct Op {
  static constexpr int bits = Fmt<F>::bits;
  static constexpr int RB = KS * bits / 8;  // bytes of one row per K-step
  static constexpr int CH = RB / 16;        // 16-byte chunks per row per K-step
  static constexpr int PITCH = RB + 16;     // LDS row pitch (padded)
  static constexpr int PANEL = 256 * PITCH; // LDS bytes of one panel
};

template <int FA, int FB> struct GemmLds {
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = Op<FA>::PANEL;
  static constexpr int SA_OFF = B_OFF + Op<FB>::PANEL;
  static constexpr int SB_OFF = SA_OFF + 256 * 4;
  static constexpr int STAGE = SB_OFF + 256 * 4;
  static constexpr int TOTAL = 2 * STAGE;
};

// Global -> register staging for one K-step panel (A or B).
template <int F> struct PanelRegs { uint4 c[Op<F>::CH]; uint32_t s; };

template <int F>
__device__ __forceinline__ void load_panel(PanelRegs<F>& R, const uint8_t* q, const uint8_t* s,
                                           int64_t rows, int64_t row0, int64_t rowbytes,
                                           int64_t nblk, int64_t k0, int tid) {
  using O = Op<F>;
  const int64_t kbyte0 = k0 * O::bits / 8;
#pragma unroll
  for (int p = 0; p < O::CH; p++) {
    const int id = p * 256 + tid;
    const int r = id / O::CH, ch = id % O::CH;
    const int64_t grow = row0 + r;
    const int64_t kb = kbyte0 + 16 * ch;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (grow < rows) {
      const uint8_t* src = q + grow * rowbytes + kb;
      if (O::bits == 6 && (rowbytes & 15)) {  // FP6 rows only 8-byte aligned
        if (kb < rowbytes) {
          const uint2 h0 = *(const uint2*)src;
          const uint2 h1 = kb + 16 <= rowbytes ? *(const uint2*)(src + 8) : make_uint2(0, 0);
          v = make_uint4(h0.x, h0.y, h1.x, h1.y);
        }
      } else if (kb + 16 <= rowbytes) {
        v = *(const uint4*)src;
      } else if (kb < rowbytes) {  // FP6 tail: half a chunk is in range
        const uint2 h = *(const uint2*)src;
        v = make_uint4(h.x, h.y, 0, 0);
      }
    }
    R.c[p] = v;
  }
  // scale bytes of row tid for the four blocks of this K-step; blocks past K
  // and rows past the end get 127 (their elements are zero)
  uint32_t sv = 0x7F7F7F7Fu;
  const int64_t grow = row0 + tid;
  if (grow < rows) {
    const int64_t b0 = k0 / 32;
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const uint32_t byte = (b0 + b < nblk) ? s[grow * nblk + b0 + b] : 0x7Fu;
      w |= byte << (8 * b);
    }
    sv = w;
  }
  R.s = sv;
}

template <int F>
__device__ __forceinline__ void store_panel(const PanelRegs<F>& R, uint8_t* panel, uint8_t* sp,
                                            int tid) {
  using O = Op<F>;
#pragma unroll
  for (int p = 0; p < O::CH; p++) {
    const int id = p * 256 + tid;
    const int r = id / O::CH, ch = id % O::CH;
    *(uint4*)(panel + r * O::PITCH + 16 * ch) = R.c[p];
  }
  *(uint32_t*)(sp + 4 * tid) = R.s;
}

// Operand of one 16-row tile for this lane (row = lane % 16 of the tile, block kb).
template <int F>
__device__ __forceinline__ v8i read_operand(const uint8_t* panel, int row, int kb) {
  using O = Op<F>;
  const uint8_t* base = panel + row * O::PITCH;
  v8i v = {0, 0, 0, 0, 0, 0, 0, 0};
  if (O::bits == 8) {
    const uint4 a = *(const uint4*)(base + 16 * kb);
    const uint4 b = *(const uint4*)(base + 64 + 16 * kb);
    v[0] = (int)a.x; v[1] = (int)a.y; v[2] = (int)a.z; v[3] = (int)a.w;
    v[4] = (int)b.x; v[5] = (int)b.y; v[6] = (int)b.z; v[7] = (int)b.w;
  } else if (O::bits == 4) {
    const uint4 a = *(const uint4*)(base + 16 * kb);
    v[0] = (int)a.x; v[1] = (int)a.y; v[2] = (int)a.z; v[3] = (int)a.w;
  } else {
    const uint2 a = *(const uint2*)(base + 24 * kb);
    const uint2 b = *(const uint2*)(base + 24 * kb + 8);
    const uint2 c = *(const uint2*)(base + 24 * kb + 16);
    v[0] = (int)a.x; v[1] = (int)a.y; v[2] = (int)b.x; v[3] = (int)b.y;
    v[4] = (int)c.x; v[5] = (int)c.y;
  }
  return v;
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN), by the
// hardware conversion; fp32 subnormals are kept.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
__device__ __forceinline__ uint16_t bf16_bits(float a) {
  return __builtin_bit_cast(uint16_t, (__bf16)a);
}

// BF16OUT: C as bf16 at cb (else fp32 at c); one epilogue per instantiation.
template <int FA, int FB, bool BF16OUT>
__global__ __launch_bounds__(256) void k_gemm(const uint8_t* __restrict__ aq,
                                              const uint8_t* __restrict__ as,
                                              const uint8_t* __restrict__ bq,
                                              const uint8_t* __restrict__ bs, int64_t M,
                                              int64_t N, int64_t K, float* __restrict__ c,
                                              uint16_t* __restrict__ cb, int64_t ldc, int tiles_n) {
  using L = GemmLds<FA, FB>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[L::TOTAL];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t arow = K * Op<FA>::bits / 8, brow = K * Op<FB>::bits / 8;
  const int64_t nblk = K / 32;
  const int nk = (int)((K + KS - 1) / KS);
  const int lr = lane & 15, kb = lane >> 4;

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 8; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  PanelRegs<FA> ra;
  PanelRegs<FB> rb;
  load_panel<FA>(ra, aq, as, M, m0, arow, nblk, 0, tid);
  load_panel<FB>(rb, bq, bs, N, n0, brow, nblk, 0, tid);
  store_panel<FA>(ra, lds + L::A_OFF, lds + L::SA_OFF, tid);
  store_panel<FB>(rb, lds + L::B_OFF, lds + L::SB_OFF, tid);
  __syncthreads();

  for (int ks = 0; ks < nk; ks++) {
    const int cur = ks & 1;
    uint8_t* st = lds + cur * L::STAGE;
    if (ks + 1 < nk) {
      load_panel<FA>(ra, aq, as, M, m0, arow, nblk, (int64_t)(ks + 1) * KS, tid);
      load_panel<FB>(rb, bq, bs, N, n0, brow, nblk, (int64_t)(ks + 1) * KS, tid);
    }
    v8i bop[8];
    int bsc[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int row = wn * 128 + j * 16 + lr;
      bop[j] = read_operand<FB>(st + L::B_OFF, row, kb);
      bsc[j] = st[L::SB_OFF + row * 4 + kb];
    }
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int row = wm * 128 + i * 16 + lr;
      const v8i aop = read_operand<FA>(st + L::A_OFF, row, kb);
      const int asc = st[L::SA_OFF + row * 4 + kb];
#pragma unroll
      for (int j = 0; j < 8; j++)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[j], acc[i][j], FA, FB,
                                                                     0, asc, 0, bsc[j]);
    }
    if (ks + 1 < nk) {
      uint8_t* nx = lds + (cur ^ 1) * L::STAGE;
      store_panel<FA>(ra, nx + L::A_OFF, nx + L::SA_OFF, tid);
      store_panel<FB>(rb, nx + L::B_OFF, nx + L::SB_OFF, tid);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 8; i++) {
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int64_t col = n0 + wn * 128 + j * 16 + lr;
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int64_t row = m0 + wm * 128 + i * 16 + 4 * kb + v;
        if (row < M && col < N) {
          if (BF16OUT)
            cb[row * ldc + col] = bf16_bits(acc[i][j][v]);
          else
            c[row * ldc + col] = acc[i][j][v];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MXINT8 x MXINT8
// ---------------------------------------------------------------------------
// gfx950's block-scaled matrix instruction takes no integer elements.  An
// MXINT8 element n / 64 times its block scale 2^(s - 127) is n * 2^(s - 133):
// an integer of at most 7 significant bits times a power of two, which bf16
// holds exactly (8 significant bits) at or above 2^-126; below that (scale
// codes under 7) it is a multiple of 2^-133, bf16's subnormal step, so it is
// exact as a subnormal.  The conversion and the bf16 instruction keep
// subnormals, so every product is exact whatever the other operand's scale.
// So each lane turns its operand bytes into bf16 with the scale folded in, and
// a bf16 matrix instruction with K = 32 -- one block per instruction -- forms
// the products exactly and accumulates them in fp32.  Folding the scale into
// the operands costs one conversion per operand element per tile pass; an
// integer instruction would instead need a per-output fp32 rescale after every
// block, which the vector ALU cannot keep up with.
// 8 INT8 codes (w: bytes 0..7 = elements 0..7) of one block with scale code
// s, as bf16 values n * 2^(s - 133).
__device__ __forceinline__ v8bf i8_bf16(uint2 w, int s) {
  const int e = s - 133;
  float f[8];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    f[k] = __builtin_amdgcn_ldexpf((float)(int)(int8_t)(w.x >> (8 * k)), e);
    f[4 + k] = __builtin_amdgcn_ldexpf((float)(int)(int8_t)(w.y >> (8 * k)), e);
  }
  const uint4 p = make_uint4(bf16x2_bits(f[0], f[1]), bf16x2_bits(f[2], f[3]),
                             bf16x2_bits(f[4], f[5]), bf16x2_bits(f[6], f[7]));
  return __builtin_bit_cast(v8bf, p);
}

// Same tiling and staging as k_gemm (256 x 256 tile, four waves of 128 x 128,
// K-steps of four blocks through two LDS stages); per block one 16x16x32 bf16
// instruction per 16 x 16 output tile.  Lane l supplies row l % 16 of its
// operand tile, elements 8 (l / 16) .. 8 (l / 16) + 7 of the block.
// (a template only so that the units of other formats do not compile it)
template <int I8, bool BF16OUT>
__global__ __launch_bounds__(256) void k_gemm_i8(const uint8_t* __restrict__ aq,
                                                 const uint8_t* __restrict__ as,
                                                 const uint8_t* __restrict__ bq,
                                                 const uint8_t* __restrict__ bs, int64_t M,
                                                 int64_t N, int64_t K, float* __restrict__ c,
                                                 uint16_t* __restrict__ cb, int64_t ldc,
                                                 int tiles_n) {
  using L = GemmLds<INT8, INT8>;
  using O = Op<INT8>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[L::TOTAL];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t nblk = K / 32;
  const int nk = (int)((K + KS - 1) / KS);
  const int lr = lane & 15, kg = lane >> 4;

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 8; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  PanelRegs<INT8> ra, rb;
  load_panel<INT8>(ra, aq, as, M, m0, K, nblk, 0, tid);
  load_panel<INT8>(rb, bq, bs, N, n0, K, nblk, 0, tid);
  store_panel<INT8>(ra, lds + L::A_OFF, lds + L::SA_OFF, tid);
  store_panel<INT8>(rb, lds + L::B_OFF, lds + L::SB_OFF, tid);
  __syncthreads();

  for (int ks = 0; ks < nk; ks++) {
    const int cur = ks & 1;
    uint8_t* st = lds + cur * L::STAGE;
    if (ks + 1 < nk) {
      load_panel<INT8>(ra, aq, as, M, m0, K, nblk, (int64_t)(ks + 1) * KS, tid);
      load_panel<INT8>(rb, bq, bs, N, n0, K, nblk, (int64_t)(ks + 1) * KS, tid);
    }
    // one block at a time keeps one block's converted operands live
#pragma unroll 1
    for (int b = 0; b < KS / 32; b++) {
      v8bf bop[8];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int row = wn * 128 + j * 16 + lr;
        const uint2 w = *(const uint2*)(st + L::B_OFF + row * O::PITCH + 32 * b + 8 * kg);
        bop[j] = i8_bf16(w, st[L::SB_OFF + row * 4 + b]);
      }
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int row = wm * 128 + i * 16 + lr;
        const uint2 w = *(const uint2*)(st + L::A_OFF + row * O::PITCH + 32 * b + 8 * kg);
        const v8bf aop = i8_bf16(w, st[L::SA_OFF + row * 4 + b]);
#pragma unroll
        for (int j = 0; j < 8; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[j], acc[i][j], 0, 0, 0);
      }
    }
    if (ks + 1 < nk) {
      uint8_t* nx = lds + (cur ^ 1) * L::STAGE;
      store_panel<INT8>(ra, nx + L::A_OFF, nx + L::SA_OFF, tid);
      store_panel<INT8>(rb, nx + L::B_OFF, nx + L::SB_OFF, tid);
    }
    __syncthreads();
  }

  // lane l holds C[4 (l / 16) + v][l % 16] of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < 8; i++) {
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int64_t col = n0 + wn * 128 + j * 16 + lr;
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int64_t row = m0 + wm * 128 + i * 16 + 4 * kg + v;
        if (row < M && col < N) {
          if (BF16OUT)
            cb[row * ldc + col] = bf16_bits(acc[i][j][v]);
          else
            c[row * ldc + col] = acc[i][j][v];
        }
      }
    }
  }
}

template <int I8 = INT8>
static hipError_t gemm_i8_launch(const void* aq, const uint8_t* as, const void* bq,
                                 const uint8_t* bs, int64_t M, int64_t N, int64_t K, float* c,
                                 int64_t ldc, int out_fmt, uint8_t* out_q, hipStream_t st) {
  if (out_fmt >= 0 && out_fmt != GEMM_OUT_BF16) return hipErrorNotSupported;
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  if (out_fmt == GEMM_OUT_BF16)
    hipLaunchKernelGGL((k_gemm_i8<I8, true>), dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, st,
                       (const uint8_t*)aq, as, (const uint8_t*)bq, bs, M, N, K, c, (uint16_t*)out_q, ldc,
                       (int)tiles_n);
  else
    hipLaunchKernelGGL((k_gemm_i8<I8, false>), dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, st,
                       (const uint8_t*)aq, as, (const uint8_t*)bq, bs, M, N, K, c, nullptr, ldc,
                       (int)tiles_n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// staged kernel (K % 512 == 0, scale arrays 16-byte aligned, operands < 4 GiB)
//
// Persistent: the grid holds one workgroup per compute unit (at most one fits:
// it takes the whole LDS and all registers of its SIMDs), and workgroup b
// computes the 256 x 256 tiles b, b + G, b + 2G, ... of C (G workgroups).  Per
// stage of KS elements of K (256 when both operands are FP4, so that every
// operand row of a stage is one 128-byte line; else 128) the A and B panels
// (256 rows each) go global -> LDS directly (buffer_load ... lds; rows past the
// matrix edge fall outside the buffer and read zero) into a ring of NST
// stages, issued NST - 1 stages ahead.  The stages of a workgroup's tiles form
// one stream: the last stages of a tile load the first stages of its next
// tile, so the ring never drains between tiles.  Panel rows are stored
// unpadded with their 16-byte chunks XOR-swizzled so that the rows read at one
// K offset hit distinct LDS banks.  The E8M0 scales travel separately, 32
// bytes (1024 elements of K) per row at a time, into two alternating LDS
// buffers: one 16-byte load per lane pair and row instead of a few bytes per
// row and stage, the loads of a chunk either with its first stage or (SPREAD)
// one per stage over the stages before it.  Every offset that can reach past a matrix (rows past M or N,
// the last scale chunk of a row) is in the range-checked VGPR offset of its
// load, relative to a buffer resource that starts at the tile.
//
// Four waves own 128 x 128 pieces of the tile, with their accumulators in the
// AGPR file.  A stage is SUB substeps of 64 elements of K (one
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 deep); each wave issues a substep's 16
// instructions with the LDS reads of a later substep's operands slotted in
// between them (a ring of operand registers), so the matrix unit is fed
// while those operands arrive.  One barrier per stage, as soon as the stage's
// operands are all read, hands the ring slot back to the loads, which are
// then spread over the rest of the stage.
//
// The first substep of a tile starts its sums from zero (the instruction's
// accumulator operand is the constant 0) and, for fp32 and bf16 output, stores
// the previous tile's results piece by piece just before each instruction
// overwrites them, so C leaves while the matrix unit works on the next tile.
// The output kind is a template parameter: each instantiation carries one
// epilogue.
// ---------------------------------------------------------------------------
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int LDS_MAX = 160 * 1024;

template <int FA, int FB, int KS_> struct Fast {
  static constexpr int KS = KS_;                      // K elements per stage
  static constexpr int SUB = KS / 64;                 // 32x32x64 substeps per stage
  static constexpr int RBA = KS * Fmt<FA>::bits / 8;  // bytes per operand row per stage
  static constexpr int RBB = KS * Fmt<FB>::bits / 8;
  static constexpr int CHA = RBA / 16, CHB = RBB / 16;  // 16-byte chunks per row
  static constexpr int A_OFF = 0, B_OFF = 256 * RBA;
  static constexpr int STAGE = 256 * (RBA + RBB);
  static constexpr int SC_ROW = 32;                   // scale bytes per row per chunk
  static constexpr int SPC = SC_ROW * 32 / KS;        // stages per scale chunk
  static constexpr int SC_BUF = 512 * SC_ROW;         // one chunk: 256 A rows, then 256 B rows
  static constexpr int NST0 = (LDS_MAX - 2 * SC_BUF) / STAGE;
  static constexpr int NST = NST0 > 4 ? 4 : NST0;
  static constexpr int SC_OFF = NST * STAGE;
  static constexpr int TOTAL = SC_OFF + 2 * SC_BUF;
  static_assert(NST >= 2 && SPC >= NST, "stage ring and scale buffers");
  // spread scale loads: the last of a chunk's four must land before its first
  // stage
  static_assert(SPC % 4 == 0 && NST - 1 <= SPC / 4, "spread scale loads");
};

template <int CH>
__device__ __forceinline__ int swz(int r) {
  if (CH == 8) return (r >> 1) & 7;  // 128-byte rows
  if (CH == 4) return (r >> 2) & 3;  // 64-byte rows
  return 0;                          // 96-byte FP6 rows: unswizzled
}

// dma16 for the lanes of `exec` when `on` is nonzero, else for no lane.
__device__ __forceinline__ void dma16_if(v4i rs, uint32_t voff, uint32_t soff, uint32_t lds_dst,
                                         int on) {
  uint64_t saved;
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_mov_b64 %0, exec\n\t"
      "s_cmp_lg_u32 %5, 0\n\t"
      "s_cselect_b64 exec, exec, 0\n\t"
      "buffer_load_dwordx4 %1, %2, %4 offen lds\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rs), "s"(lds_dst), "s"(soff), "s"(__builtin_amdgcn_readfirstlane(on))
      : "memory", "m0", "scc");
}

// Workgroup barrier as one asm block with a memory clobber: the compiler can
// neither move LDS accesses across it nor add waits of its own.  The
// scheduling fences keep the matrix instructions (not memory operations, so
// unaffected by the clobber) on their side of it.
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" : : : "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// Barrier after this wave's buffer->LDS loads are down to at most n in flight
// and its own LDS reads are back.
template <int n>
__device__ __forceinline__ void wait_all_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(n) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Operand of one 32-row tile for substep u of a stage: lane l = row l % 32 of
// the tile, block kb = l / 32 of the substep.  FP8 lanes hold the 16-byte
// pieces at K offsets 16 kb and 32 + 16 kb of the substep; FP6 / FP4 lanes
// hold their block.  `lb` points at the lane's row, whose chunks are swizzled
// with `sw`.
template <int F, int CH>
__device__ __forceinline__ v8i read32(const uint8_t* lb, int toff, int u, int kb, int sw) {
  constexpr int bits = Fmt<F>::bits;
  const uint8_t* base = lb + toff;
  v8i v = {0, 0, 0, 0, 0, 0, 0, 0};
  if (bits == 8) {
    const uint4 a = *(const uint4*)(base + 16 * ((4 * u + kb) ^ sw));
    const uint4 b = *(const uint4*)(base + 16 * ((4 * u + 2 + kb) ^ sw));
    v[0] = (int)a.x; v[1] = (int)a.y; v[2] = (int)a.z; v[3] = (int)a.w;
    v[4] = (int)b.x; v[5] = (int)b.y; v[6] = (int)b.z; v[7] = (int)b.w;
  } else if (bits == 4) {
    const uint4 a = *(const uint4*)(base + 16 * ((2 * u + kb) ^ sw));
    v[0] = (int)a.x; v[1] = (int)a.y; v[2] = (int)a.z; v[3] = (int)a.w;
  } else {
    const uint8_t* q = base + 24 * (2 * u + kb);
    const uint2 a = *(const uint2*)q;
    const uint2 b = *(const uint2*)(q + 8);
    const uint2 c = *(const uint2*)(q + 16);
    v[0] = (int)a.x; v[1] = (int)a.y; v[2] = (int)b.x; v[3] = (int)b.y;
    v[4] = (int)c.x; v[5] = (int)c.y;
  }
  return v;
}

// Tile `local` of a rows x cols block of tiles starting at (r0, c0), walked in
// groups of 4 tile rows so that tiles running together share A and B panels.
__device__ __forceinline__ void walk_block(int local, int rows, int cols, int r0, int c0, int& tm,
                                           int& tn) {
  constexpr int GROUP_M = 4;
  const int per_group = GROUP_M * cols;
  const int g = local / per_group;
  const int first_m = g * GROUP_M;
  const int gm = rows - first_m < GROUP_M ? rows - first_m : GROUP_M;
  const int w = local % per_group;
  tm = r0 + first_m + w % gm;
  tn = c0 + w / gm;
}

// Workgroup -> C tile.  Workgroups are dispatched to the 8 XCDs round-robin;
// give each XCD a contiguous range of tiles, walked in groups of GROUP_M tile
// rows so that concurrently running tiles share A and B panels in its L2.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GROUP_M = 4;
  const int T = tiles_m * tiles_n;
  const int q = T / 8, r = T % 8;
  const int x = bid % 8, local = bid / 8;
  const int lin = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
  const int per_group = GROUP_M * tiles_n;
  const int g = lin / per_group;
  const int first_m = g * GROUP_M;
  const int gm = tiles_m - first_m < GROUP_M ? tiles_m - first_m : GROUP_M;
  const int w = lin % per_group;
  tm = first_m + w % gm;
  tn = w / gm;
}

// Operands of one 64-element substep for one wave: 4 A tiles and 4 B tiles of
// 32 rows, with their scale bytes.
struct Ops {
  v8i a[4], b[4];
  int sa[4], sb[4];
};

// Where a wave's operands sit in LDS: its rows' offsets and swizzles.
struct Lanes {
  int arow, brow;  // first A / B row of the wave's tiles for this lane
  int kb, swa, swb;
  int bsh[2];      // bit offset of the lane's scale byte in a word, even / odd substep
};

// The scale bytes of one stage for the wave's 8 tiles: KS / 32 bytes per row
// (one or two dwords), read once per stage from chunk buffer `par` at byte
// offset `off` of each row's 32.  A chunk buffer holds blocks of 32 rows, each
// as [16-byte half][row][16 bytes], so the 32 rows a read takes sit 16 bytes
// apart (two rows to a bank) instead of 32.
template <int KS> struct ScaleWords {
  uint32_t a[4][KS / 128], b[4][KS / 128];
};

template <class C>
__device__ __forceinline__ void read_scale_words(ScaleWords<C::KS>& sw, const uint8_t* lds, int par,
                                                 int off, const Lanes& w) {
  const uint8_t* sc = lds + C::SC_OFF + par * C::SC_BUF + (off >> 4) * 512 + (off & 15);
  const uint8_t* sa = sc + (w.arow >> 5) * 1024 + (w.arow & 31) * 16;
  const uint8_t* sb = sc + (8 + (w.brow >> 5)) * 1024 + (w.brow & 31) * 16;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint8_t* pa = sa + 1024 * i;
    const uint8_t* pb = sb + 1024 * i;
    if (C::KS == 256) {
      const uint2 x = *(const uint2*)pa, y = *(const uint2*)pb;
      sw.a[i][0] = x.x; sw.a[i][C::KS / 128 - 1] = x.y;
      sw.b[i][0] = y.x; sw.b[i][C::KS / 128 - 1] = y.y;
    } else {
      sw.a[i][0] = *(const uint32_t*)pa;
      sw.b[i][0] = *(const uint32_t*)pb;
    }
  }
}

// Scale operands of substep u: byte 2u + kb of the stage's bytes of the row.
// For MXINT8 (I8) both of the substep's scale bytes, 2u and 2u + 1, as the
// low 16 bits: a lane's operand bytes come from both of its blocks.
template <int KS, bool I8 = false>
__device__ __forceinline__ void scales_of(Ops& o, const ScaleWords<KS>& sw, int u, const Lanes& w) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    if (I8) {
      o.sa[i] = (int)__builtin_amdgcn_ubfe(sw.a[i][u / 2], 16 * (u & 1), 16);
      o.sb[i] = (int)__builtin_amdgcn_ubfe(sw.b[i][u / 2], 16 * (u & 1), 16);
    } else {
      o.sa[i] = (int)__builtin_amdgcn_ubfe(sw.a[i][u / 2], w.bsh[u & 1], 8);
      o.sb[i] = (int)__builtin_amdgcn_ubfe(sw.b[i][u / 2], w.bsh[u & 1], 8);
    }
  }
}

// One tile's operand of substep u (t < 4: A tile t, else B tile t - 4).
template <class C, int FA, int FB>
__device__ __forceinline__ void read_tile(Ops& o, const uint8_t* st, int u, int t, const Lanes& w) {
  if (t < 4)
    o.a[t] = read32<FA, C::CHA>(st + C::A_OFF + (w.arow + 32 * t) * C::RBA, 0, u, w.kb, w.swa);
  else
    o.b[t - 4] = read32<FB, C::CHB>(st + C::B_OFF + (w.brow + 32 * (t - 4)) * C::RBB, 0, u, w.kb, w.swb);
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1: a loop whose index
// is a compile-time constant in the body however large the body is.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// One substep: the 16 block-scaled instructions on `cur`, each preceded by
// `pre(k)` and followed by `slot(k)` (LDS reads of the next substep's
// operands, the barrier, loads), in exactly this order (scheduling fences).
// With ZERO the instructions start from zero instead of adding to acc.  B is
// the instruction's first operand, so a lane's results are four consecutive
// columns of C.
template <int FA, int FB, bool ZERO, class Pre, class Slot>
__device__ __forceinline__ void substep(v16f (&acc)[4][4], const Ops& cur, Pre&& pre, Slot&& slot) {
  static_for<16>([&](auto K) {
    constexpr int k = decltype(K)::value, i = k >> 2, j = k & 3;
    pre(K);
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur.b[j], cur.a[i],
                                                                ZERO ? v16f{} : acc[i][j], FB, FA,
                                                                0, cur.sb[j], 0, cur.sa[i]);
    slot(K);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// One MXINT8 substep on the same operand registers: a lane's 32 bytes are 16
// of block 2u (K offsets 16 kb ..) and 16 of block 2u + 1 (32 + 16 kb ..).
// Four slices t of 8 bytes each become bf16 with their block's scale folded
// in (i8_bf16) and feed 16 bf16 32x32x16 instructions.  A and B lanes take
// the same K positions in the same slice, so the four slices together cover
// the substep's 64 products of every (row, column) pair exactly once, in a
// different order from the block-scaled instruction.  pre(k) precedes the
// first slice's instruction k; slot(k) follows every fourth instruction, in
// order.  With ZERO the first slice starts from zero.
template <bool ZERO, class Pre, class Slot>
__device__ __forceinline__ void substep_i8(v16f (&acc)[4][4], const Ops& cur, Pre&& pre, Slot&& slot) {
  auto convert = [&](int t, v8bf (&a8)[4], v8bf (&b8)[4]) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int sa = t < 2 ? (cur.sa[i] & 0xFF) : ((cur.sa[i] >> 8) & 0xFF);
      const int sb = t < 2 ? (cur.sb[i] & 0xFF) : ((cur.sb[i] >> 8) & 0xFF);
      a8[i] = i8_bf16(make_uint2((uint32_t)cur.a[i][2 * t], (uint32_t)cur.a[i][2 * t + 1]), sa);
      b8[i] = i8_bf16(make_uint2((uint32_t)cur.b[i][2 * t], (uint32_t)cur.b[i][2 * t + 1]), sb);
    }
  };
  // the operands of slice t + 1 are converted within slice t's last group of
  // instructions, where the scheduler can place them under the matrix work
  v8bf a8[2][4], b8[2][4];
  convert(0, a8[0], b8[0]);
  static_for<4>([&](auto T) {
    constexpr int t = decltype(T)::value, c = t & 1;
    static_for<16>([&](auto K) {
      constexpr int k = decltype(K)::value, i = k >> 2, j = k & 3;
      if constexpr (k == 12 && t < 3) convert(t + 1, a8[c ^ 1], b8[c ^ 1]);
      if constexpr (t == 0) pre(K);
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b8[c][j], a8[c][i],
                                                          ZERO && t == 0 ? v16f{} : acc[i][j], 0, 0, 0);
      if constexpr (k % 4 == 3) slot(std::integral_constant<int, 4 * t + k / 4>{});
    });
  });
}

// Element k of an accumulator tile as fp32 bits, read from its accumulation
// register at this point of the program.  Left to itself the compiler copies
// every accumulator of the epilogue into vector registers at its start, which
// for 256 values spills; a read in the asm keeps each value in place until it
// is used.  The compiler does not count wait states for asm, so the first
// such read must follow acc_settle: a read of an accumulator needs 18 wait
// states after the 16-pass matrix instruction that wrote it.  Both are
// volatile, which keeps them in program order.
__device__ __forceinline__ uint32_t acc_bits(const v16f& t, int k) {
  uint32_t r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(t[k]));
  return r;
}
__device__ __forceinline__ void acc_settle() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory"); }

// MX output of the product: C row-wise in MX format, blocks of 32 along N
// (Algorithm 1 of the MX summary, section 3, applied to each fp32 block of the
// product, round to nearest even), as "Format-Aware Fusion for Fast FP4
// Pretraining" fuses the quantization into the producer.
struct MxOut {
  int fmt;         // E4M3, E5M2 or E2M1
  uint8_t* q;      // [M x N_p] packed codes (N_p: N padded to whole blocks)
  uint8_t* s;      // [M x N_p/32] scales
};

// A wave's 128 x 128 piece (rows r0.., columns c0.., c0 % 128 == 0) as MX
// blocks: the 32 columns of acc[i][j] for row 32 i + l % 32 are one block,
// held half by lane l (columns 8 q + 4 (l / 32) + e, q and e in 0..3) and half
// by lane l ^ 32.  The block max and the codes' halves are exchanged between
// the two lanes, so each lane stores 16 consecutive columns' codes in one
// piece.  Each step runs over the four tiles of a tile row at once, without
// per-tile branches, so the exchanges of different tiles overlap: the
// hardware conversion is applied to every block and replaced afterwards, on
// the rare lanes that need it, by the exact conversion (scale codes below
// DazFree) or the NaN codes.
template <int F>
__device__ __forceinline__ void store_mx(const v16f (&acc)[4][4], const MxOut& mo, int64_t r0, int64_t c0,
                                         int64_t M, int64_t N, int lane) {
  constexpr int bits = Fmt<F>::bits;
  const int lr = lane & 31, hi = lane >> 5;
  const int partner = (lane ^ 32) << 2;
  const int64_t nb = (N + 31) >> 5;  // blocks per row; a short last block is padded
  const int64_t blk0 = c0 >> 5;
  const bool s_dword = (nb & 3) == 0 && ((uintptr_t)mo.s & 3) == 0 && blk0 + 3 < nb;
  acc_settle();
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int64_t row = r0 + 32 * i + lr;
    // the element values of tile (i, j) as fp32 bits, read from the
    // accumulation registers where they are used (acc_bits)
    auto vals = [&](int j, int k0, uint32_t (&v)[8]) {
#pragma unroll
      for (int k = 0; k < 8; k++) v[k] = acc_bits(acc[i][j], k0 + k);
    };
    uint32_t code[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      uint32_t am = 0;
#pragma unroll
      for (int k = 0; k < 16; k++) am = umax(am, acc_bits(acc[i][j], k) & 0x7FFFFFFFu);
      code[j] = am;
    }
#pragma unroll
    for (int j = 0; j < 4; j++)
      code[j] = scale_code<F>(umax(code[j], (uint32_t)__builtin_amdgcn_ds_bpermute(partner, (int)code[j])));
    Pack8 p[4][2];
    bool slow = false;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      uint32_t v[8];
      vals(j, 0, v);
      p[j][0] = hw_convert8<F>(v, code[j]);
      vals(j, 8, v);
      p[j][1] = hw_convert8<F>(v, code[j]);
      slow |= !hw_ok<F>(code[j]);
    }
    if (slow) {
      uint32_t rnd[8];
#pragma unroll
      for (int j = 0; j < 4; j++)
        if (!hw_ok<F>(code[j])) {
          uint32_t v[8];
          vals(j, 0, v);
          p[j][0] = convert8<F, false>(v, code[j], rnd);
          vals(j, 8, v);
          p[j][1] = convert8<F, false>(v, code[j], rnd);
        }
    }
    // codes of this lane's columns: groups q = 0..3 of four, at 8 q + 4 hi;
    // p[j][0] holds groups 0, 1 and p[j][1] groups 2, 3.  The values to send
    // are fixed in registers before the exchanges, so the per-lane choice
    // cannot become branches around them.
    uint32_t x[4][2];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if (bits == 8) {
        // the low lane keeps groups 0-1 of both lanes (columns 0-15), the
        // high lane groups 2-3 (columns 16-31)
        uint32_t s1 = hi ? p[j][0].w[0] : p[j][1].w[0];
        uint32_t s2 = hi ? p[j][0].w[1] : p[j][1].w[1];
        asm volatile("" : "+v"(s1), "+v"(s2));
        x[j][0] = (uint32_t)__builtin_amdgcn_ds_bpermute(partner, (int)s1);
        x[j][1] = (uint32_t)__builtin_amdgcn_ds_bpermute(partner, (int)s2);
      } else {  // E2M1: group q is 16 bits (w[0]: groups 0 | 1 << 16 or 2 | 3 << 16)
        uint32_t s1 = hi ? p[j][0].w[0] : p[j][1].w[0];
        asm volatile("" : "+v"(s1));
        x[j][0] = (uint32_t)__builtin_amdgcn_ds_bpermute(partner, (int)s1);
      }
    }
    const bool rlive = row < M;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int64_t blk = blk0 + j;
      const bool live = rlive && blk < nb;
      if (bits == 8) {
        const uint32_t g0 = p[j][0].w[0], g1 = p[j][0].w[1];
        const uint32_t g2 = p[j][1].w[0], g3 = p[j][1].w[1];
        const uint32_t r1 = x[j][0], r2 = x[j][1];
        const uint4 o = hi ? make_uint4(r1, g2, r2, g3) : make_uint4(g0, r1, g1, r2);
        if (live) *(uint4*)(mo.q + row * (32 * nb) + 32 * blk + 16 * hi) = o;
      } else {
        const uint32_t r = x[j][0];
        const uint32_t own = hi ? p[j][1].w[0] : p[j][0].w[0];
        uint2 o;
        if (hi) {  // columns 16-31: groups 2 (partner, own), 3 (partner, own)
          o.x = (r & 0xFFFFu) | (own << 16);
          o.y = (r >> 16) | (own & 0xFFFF0000u);
        } else {  // columns 0-15: groups 0 (own, partner), 1 (own, partner)
          o.x = (own & 0xFFFFu) | (r << 16);
          o.y = (own >> 16) | (r & 0xFFFF0000u);
        }
        if (live) *(uint2*)(mo.q + row * (16 * nb) + 16 * blk + 8 * hi) = o;
      }
    }
    // scales: both lanes of a row hold its four codes; the low lane stores
    // them, as one dword where the row's scale offset is 4-byte aligned
    if (rlive && hi == 0) {
      uint8_t* sp = mo.s + row * nb + blk0;
      if (s_dword) {
        *(uint32_t*)sp = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
      } else {
#pragma unroll
        for (int j = 0; j < 4; j++)
          if (blk0 + j < nb) sp[j] = (uint8_t)code[j];
      }
    }
  }
}

// Output kinds of the staged kernel.
enum { OUT_F32 = 0, OUT_BF16 = 1, OUT_MX_E4M3 = 2, OUT_MX_E5M2 = 3, OUT_MX_E2M1 = 4 };
template <int OUT> struct OutMx { static constexpr int fmt = OUT == OUT_MX_E4M3 ? E4M3 : (OUT == OUT_MX_E5M2 ? E5M2 : E2M1); };

struct FastArgs {
  const uint8_t* aq;
  const uint8_t* as;
  const uint8_t* bq;
  const uint8_t* bs;
  int64_t M, N, K;
  void* c;        // fp32 C, bf16 C, or MX codes
  uint8_t* cs;    // MX scales
  int64_t ldc;    // fp32 / bf16 C: row pitch in elements
  int tiles_m, tiles_n;
  int vec;        // fp32 / bf16 C: 16 / 8-byte stores allowed (pointer and pitch aligned)
  // XCD blocks: with part_m * part_n == 8 (and one workgroup per compute unit,
  // G a multiple of 8), XCD x = b % 8 owns the block (x / part_n, x % part_n) of
  // a part_m x part_n split of the tile grid and walks it alone, so each XCD's
  // L2 fetches only its block's A and B panels; 0: one contiguous tile range
  // per XCD (tile_of)
  int part_m, part_n;
};

// Stores of one 32 x 32 accumulator tile acc[i][j] of a wave's 128 x 128 piece
// (rows r0 + 32 i + l % 32, columns c0 + 32 j + 8 q + 4 (l / 32) + e for
// element 4 q + e of lane l), fp32 or bf16, inside M x N.  With ASM the bf16
// values are read one accumulator at a time (acc_bits), which keeps the
// conversion's registers few while the operand ring is live; the tile must
// then not have been written by one of the last few matrix instructions.
template <int OUT, bool ASM = false>
__device__ __forceinline__ void store_tile(const v16f& t, const FastArgs& g, int64_t r0, int64_t c0,
                                           int i, int j, int lane) {
  auto val = [&](int k) {
    if constexpr (ASM) return __builtin_bit_cast(float, acc_bits(t, k));
    else return t[k];
  };
  const int64_t row = r0 + 32 * i + (lane & 31);
  if (row >= g.M) return;
  const int64_t col0 = c0 + 32 * j + 4 * (lane >> 5);
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const int64_t col = col0 + 8 * q;
    if (OUT == OUT_F32) {
      float* crow = (float*)g.c + row * g.ldc;
      if (g.vec && col + 3 < g.N) {
        *(float4*)(crow + col) = make_float4(t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; e++)
          if (col + e < g.N) crow[col + e] = t[4 * q + e];
      }
    } else {
      uint16_t* crow = (uint16_t*)g.c + row * g.ldc;
      if (g.vec && col + 3 < g.N) {
        *(uint2*)(crow + col) = make_uint2(bf16x2_bits(val(4 * q), val(4 * q + 1)),
                                           bf16x2_bits(val(4 * q + 2), val(4 * q + 3)));
      } else {
#pragma unroll
        for (int e = 0; e < 4; e++)
          if (col + e < g.N) crow[col + e] = bf16_bits(val(4 * q + e));
      }
    }
  }
}

template <int FA, int FB, int KS, int OUT, bool SPREAD>
__global__ __launch_bounds__(256) void k_gemm_fast(FastArgs g) {
  using C = Fast<FA, FB, KS>;
  constexpr int NST = C::NST, SUB = C::SUB, SPC = C::SPC;
  constexpr int SEGS = C::CHA + C::CHB;  // 1 KB panel segments per wave per stage
  constexpr int SEG_A = 4 * C::CHA;
  constexpr bool MXO = OUT >= OUT_MX_E4M3;
  // An accumulation-register operand anywhere in the kernel lets the compiler
  // place the accumulators in the AGPR file (256 of them per wave), leaving
  // the VGPRs to two substeps of operands.
  asm volatile("; uses agprs %0" : : "a"(0));
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::TOTAL];
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a wave-uniform (scalar) value: LDS destinations stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 pieces of 128 x 128
  const int64_t M = g.M, N = g.N;
  const uint32_t arow = (uint32_t)(g.K * Fmt<FA>::bits / 8), brow = (uint32_t)(g.K * Fmt<FB>::bits / 8);
  const uint32_t nblk = (uint32_t)(g.K / 32);
  const int nk = (int)(g.K / KS);                // stages per tile (>= NST)
  const int nch = (nk + SPC - 1) / SPC;          // scale chunks per tile
  const int T = g.tiles_m * g.tiles_n, G = gridDim.x, bid = blockIdx.x;
  // tiles of this workgroup: every G-th tile from bid, or every (G / 8)-th
  // tile of its XCD's block
  const int bm = g.part_m ? g.tiles_m / g.part_m : 0, bn = g.part_m ? g.tiles_n / g.part_n : 0;
  const int xcd = bid % 8, wl = bid / 8, wpx = G / 8;
  const int nt = g.part_m ? (bm * bn - 1 - wl) / wpx + 1 : (T - 1 - bid) / G + 1;

  // this wave's panel segments I = wave + 4 k (A segments first, then B);
  // lane chunk I * 64 + lane of the panel, as an offset from the tile's first
  // row
  uint32_t voff[SEGS];
  uint32_t lofs[SEGS];
  bool isb[SEGS];
#pragma unroll
  for (int k = 0; k < SEGS; k++) {
    const int I = wave + 4 * k;
    isb[k] = I >= SEG_A;
    const int Ip = isb[k] ? I - SEG_A : I;
    const int ch = isb[k] ? C::CHB : C::CHA;
    const int Lc = Ip * 64 + lane;
    const int r = Lc / ch, pc = Lc % ch;
    const int cc = pc ^ (isb[k] ? swz<C::CHB>(r) : swz<C::CHA>(r));
    voff[k] = (uint32_t)r * (isb[k] ? brow : arow) + 16 * cc;
    lofs[k] = (uint32_t)((isb[k] ? C::B_OFF : C::A_OFF) + Ip * 1024);
  }
  // scale chunks: wave w loads A scale rows 64 w .. 64 w + 63 and the same B
  // rows, 32 rows per load; lane l takes 16-byte half l / 32 of row l % 32, so
  // a 32-row block lands in LDS as [half][row][16 bytes] (read_scale_words)
  const uint32_t vs0 = (uint32_t)(wave * 64 + (lane & 31)) * nblk + 16 * (lane >> 5);
  const uint32_t vs1 = vs0 + 32 * nblk;
  const uint32_t lds0 = lds_addr(lds);
  const v4i rnone = {0, 0, 0, 0x00020000};

  // Tile t of this workgroup: its first row of A and of B (M and N past the
  // last tile, whose loads then fetch nothing).
  struct TileAt { int m0, n0; };
  auto tile_at = [&](int t) {
    TileAt r{(int)M, (int)N};
    if (t < nt) {
      int tm, tn;
      if (g.part_m)
        walk_block(wl + t * wpx, bm, bn, (xcd / g.part_n) * bm, (xcd % g.part_n) * bn, tm, tn);
      else
        tile_of(bid + t * G, g.tiles_m, g.tiles_n, tm, tn);
      r.m0 = tm * BM;
      r.n0 = tn * BN;
    }
    return r;
  };
  // Buffer resources of a tile, each starting at the tile's first row and
  // ending at the matrix's last: every row past M or N and every byte past
  // the last scale row reads zero (past the last tile they are empty).
  struct TileRs { v4i a, b, sa, sb; };
  auto tile_rs = [&](TileAt o) {
    TileRs r;
    const uint32_t mr = (uint32_t)(M - o.m0), nr = (uint32_t)(N - o.n0);
    r.a = make_rsrc(g.aq + (int64_t)o.m0 * arow, mr * arow);
    r.b = make_rsrc(g.bq + (int64_t)o.n0 * brow, nr * brow);
    r.sa = make_rsrc(g.as + (int64_t)o.m0 * nblk, mr * nblk);
    r.sb = make_rsrc(g.bs + (int64_t)o.n0 * nblk, nr * nblk);
    return r;
  };
  // Load j (0 .. NLD-1) of stage sl of the tile with resources r, into ring
  // slot `slot`: with SPREAD, j = 0 is no load here (the scale piece of the
  // stage, scale_piece); else the four scale loads of a chunk (masked off
  // except at the first stage of a chunk, so the loop body has no branch;
  // chunk buffers alternate with the workgroup's running chunk count, parity
  // `par`).  Then the panel segments.
  constexpr int NSC = SPREAD ? 1 : 4;
  constexpr int NLD = NSC + SEGS;
  auto issue_one = [&](const TileRs& r, int sl, int par, int slot, int j) {
    if (j < NSC) {
      if constexpr (!SPREAD) {
        const bool chunk = (sl % SPC) == 0;
        const uint32_t sdst = lds0 + C::SC_OFF + par * C::SC_BUF + wave * 64 * C::SC_ROW +
                              (j >> 1) * 256 * C::SC_ROW + (j & 1) * 32 * C::SC_ROW;
        const uint32_t vo = ((j & 1) ? vs1 : vs0) + (uint32_t)(sl / SPC) * C::SC_ROW;
        dma16_if(j < 2 ? r.sa : r.sb, vo, 0u, sdst, chunk);
      }
    } else {
      const int k = j - NSC;
      dma16(isb[k] ? r.b : r.a, voff[k], (uint32_t)sl * (isb[k] ? C::RBB : C::RBA),
            lds0 + (uint32_t)(slot * C::STAGE) + lofs[k]);
    }
  };
  // SPREAD (every chunk of every tile whole, at least two chunks per tile):
  // the four loads of a chunk, one per stage, SPC / 4 stages apart.  Counting
  // the chunks of the workgroup's tiles in order (chunk c in buffer c & 1),
  // load q of chunk c (A rows, then B rows; 32 rows each, then the next 32)
  // rides with the panel loads issued during stage SPC (c - 1) - 1 + q SPC / 4,
  // stages counted the same way: by then every wave has read its last scale
  // words of chunk c - 2 from that buffer (at that stage's barrier), and the
  // last load lands by the wait before chunk c's first stage, whose words are
  // read just after it (NST - 1 <= SPC / 4).  Seen from tile t, the piece
  // issued during its stage s (s < 0: the prologue, which loads chunk 0 whole
  // before) belongs to chunk cc = floor((s + 1) / SPC) + 1 of the stream of
  // chunks from tile t on: a chunk of tile t or t + 1.
  auto scale_piece = [&](int t, int s, TileAt a0, TileAt a1) {
    constexpr int GAP = SPC / 4;
    const int d = s + 1;  // >= 1 - NST >= -SPC
    const int fl = d < 0 ? -1 : d / SPC;
    const int pos = d - fl * SPC, cc = fl + 1, q = pos / GAP;
    int c = cc;
    TileAt a = a0;
    if (c >= nch) {
      c -= nch;
      a = a1;
    }
    const bool bpart = q >= 2;
    const uint32_t rows = (uint32_t)(bpart ? N - a.n0 : M - a.m0);
    const v4i rs = make_rsrc((bpart ? g.bs + (int64_t)a.n0 * nblk : g.as + (int64_t)a.m0 * nblk), rows * nblk);
    const uint32_t dst = lds0 + C::SC_OFF + ((t * nch + cc) & 1) * C::SC_BUF + wave * 64 * C::SC_ROW +
                         (q >> 1) * 256 * C::SC_ROW + (q & 1) * 32 * C::SC_ROW;
    const uint32_t vo = ((q & 1) ? vs1 : vs0) + (uint32_t)c * C::SC_ROW;
    dma16_if(rs, vo, 0u, dst, cc > 0 && pos % GAP == 0);
  };

  Lanes w;
  {
    const int lr = lane & 31;
    w.kb = lane >> 5;
    w.arow = wm * 128 + lr;
    w.brow = wn * 128 + lr;
    w.swa = swz<C::CHA>(lr);
    w.swb = swz<C::CHB>(lr);
    w.bsh[0] = 8 * w.kb;
    w.bsh[1] = 16 + 8 * w.kb;
  }

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

  // operands are read RA substeps ahead into a ring of NB register sets (NB
  // divides SUB, so the ring position of a substep is the same every stage)
  constexpr int RA = SUB >= 4 ? 2 : 1;
  constexpr int NB = SUB >= 4 ? 4 : 2;
  static_assert(SUB % NB == 0 && RA < NB, "operand register ring");
  Ops ops[NB];
  ScaleWords<KS> sw, swn;

  TileAt cur = tile_at(0), nxt = tile_at(1);
  // prologue: stages 0 .. NST-1 of the first tile in flight, wait for stage 0
  // (a wait counts panel loads only: masked-off scale loads may or may not
  // count, and where they do the wait is merely longer), then the operands of
  // its first RA substeps
  if constexpr (SPREAD) {
    const TileRs r0 = tile_rs(cur);
#pragma unroll
    for (int j = 0; j < 4; j++)
      dma16(j < 2 ? r0.sa : r0.sb, (j & 1) ? vs1 : vs0, 0u,
            lds0 + C::SC_OFF + wave * 64 * C::SC_ROW + (j >> 1) * 256 * C::SC_ROW + (j & 1) * 32 * C::SC_ROW);
  }
#pragma unroll
  for (int i = 0; i < NST; i++) {
    if constexpr (SPREAD) scale_piece(0, i - NST, cur, nxt);
#pragma unroll
    for (int j = 0; j < NLD; j++) issue_one(tile_rs(cur), i, (i / SPC) & 1, i, j);
  }
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"((NST - 1) * SEGS) : "memory");
  __builtin_amdgcn_sched_barrier(0);
  read_scale_words<C>(sw, lds, 0, 0, w);
  static_for<RA>([&](auto R) {
    constexpr int r = decltype(R)::value;
    scales_of<KS, FA == INT8>(ops[r], sw, r, w);
#pragma unroll
    for (int t = 0; t < 8; t++) read_tile<C, FA, FB>(ops[r], lds, r, t, w);
  });

  // Per stage: SUB substeps.  Substep u's instructions run on ops[u % NB]
  // while the operands of the substep RA later are read into ops[(u + RA) %
  // NB], one tile after each of instructions 0-7.  Once the last operands of
  // the stage are in (after instruction SK of substep SU), every wave waits
  // for the next stage (its own loads of it landed, its LDS reads back, then
  // the barrier: every wave is also done reading the current slot) and reads
  // the next stage's scale words; the loads of the stage NST ahead (of this
  // tile or the next) into the current slot are then spread over the
  // remaining instruction slots of the stage, while the last RA substeps read
  // the next stage's first operands.  In the last stage of the last tile the
  // operands read for the stage after it are never used.
  constexpr int AHEAD = (NST - 2) * SEGS;  // panel loads still in flight at a wait
  constexpr int SU = SUB - 1 - RA;
  constexpr int SK = 11;
  constexpr int NSLOT = (15 - SK) + 16 * (SUB - 1 - SU);  // slots after the wait
  int slot = 0;          // ring slot of the current stage
  int64_t pm0 = M, pn0 = N;  // origin of the tile whose sums are in acc (none yet)
  const int64_t wr = wm * 128, wc = wn * 128;

  auto stage = [&](auto FIRST_, int t, int s) {
    constexpr bool FIRST = decltype(FIRST_)::value;
    // the next stage, whose scale words are read at the wait
    const bool last = s + 1 == nk;
    const int pn = ((last ? t + 1 : t) * nch + (last ? 0 : s + 1) / SPC) & 1;
    const int on = ((last ? 0 : s + 1) % SPC) * (KS / 32);
    // the stage NST ahead, loaded into this stage's slot after the wait
    const bool cross = s + NST >= nk;
    const int sl = cross ? s + NST - nk : s + NST;
    const int lpar = ((cross ? t + 1 : t) * nch + sl / SPC) & 1;
    const TileRs lr = tile_rs(cross ? nxt : cur);
    const int cslot = slot, nslot = slot + 1 == NST ? 0 : slot + 1;
    if constexpr (FIRST && MXO) {
      // MX output: the previous tile's blocks go out before the first
      // instruction of this one (the conversion needs whole tile rows)
      if (t > 0) store_mx<OutMx<OUT>::fmt>(acc, MxOut{OutMx<OUT>::fmt, (uint8_t*)g.c, g.cs}, pm0 + wr,
                                           pn0 + wc, M, N, lane);
    }
    static_for<SUB>([&](auto U) {
      constexpr int u = decltype(U)::value;
      constexpr int un = (u + RA) % SUB;     // substep whose operands are read
      constexpr bool next = u + RA >= SUB;   // ... of the next stage
      Ops& nx = ops[(u + RA) % NB];
      const uint8_t* st = lds + (next ? nslot : cslot) * C::STAGE;
      auto body = [&](auto K) {
        constexpr int k = decltype(K)::value;
        if constexpr (u == SU && k == SK) {
          wait_all_barrier<AHEAD>();
          read_scale_words<C>(swn, lds, pn, on, w);
        }
        if constexpr (k < 8) read_tile<C, FA, FB>(nx, st, un, k, w);
        constexpr int gi = (u - SU) * 16 + (k - SK - 1);  // slot index after the wait
        if constexpr (gi >= 0 && gi < NSLOT) {
          static_for<NLD>([&](auto J) {
            constexpr int j = decltype(J)::value;
            if constexpr ((j * NSLOT) / NLD == gi) {
              if constexpr (SPREAD && j == 0)
                scale_piece(t, s, cur, nxt);
              else
                issue_one(lr, sl, lpar, cslot, j);
            }
          });
        }
      };
      // fp32 / bf16 output: the previous tile's results of acc[i][j] leave
      // just before this tile's first instruction on acc[i][j] replaces them
      auto pre = [&](auto K) {
        constexpr int k = decltype(K)::value;
        if constexpr (FIRST && u == 0 && !MXO)
          store_tile<OUT, OUT == OUT_BF16>(acc[k >> 2][k & 3], g, pm0 + wr, pn0 + wc, k >> 2, k & 3, lane);
      };
      if constexpr (FA == INT8)
        substep_i8<FIRST && u == 0>(acc, ops[u % NB], pre, body);
      else
        substep<FA, FB, FIRST && u == 0>(acc, ops[u % NB], pre, body);
      if constexpr (next)
        scales_of<KS, FA == INT8>(nx, swn, un, w);
      else
        scales_of<KS, FA == INT8>(nx, sw, un, w);
    });
    sw = swn;
    slot = nslot;
  };

  for (int t = 0; t < nt; t++) {
    if (t > 0) {
      pm0 = cur.m0;
      pn0 = cur.n0;
      cur = nxt;
      nxt = tile_at(t + 1);
    }
    stage(std::true_type{}, t, 0);
    for (int s = 1; s < nk; s++) stage(std::false_type{}, t, s);
  }
  // the out-of-range loads of the last stages must be done before the
  // workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" : : : "memory");

  // the last tile's results
  if constexpr (MXO) {
    store_mx<OutMx<OUT>::fmt>(acc, MxOut{OutMx<OUT>::fmt, (uint8_t*)g.c, g.cs}, cur.m0 + wr,
                              cur.n0 + wc, M, N, lane);
  } else {
    static_for<16>([&](auto K) {
      constexpr int k = decltype(K)::value;
      store_tile<OUT>(acc[k >> 2][k & 3], g, cur.m0 + wr, cur.n0 + wc, k >> 2, k & 3, lane);
      __builtin_amdgcn_sched_barrier(0);
    });
  }
}

// Compute units of the current device, looked up once per device.
inline int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int FA, int FB, int KS, int OUT, bool SPREAD = false>
static hipError_t launch_fast(const GemmCall& gc, int64_t tiles_m, int64_t tiles_n) {
  FastArgs g;
  g.aq = (const uint8_t*)gc.aq;
  g.as = gc.as;
  g.bq = (const uint8_t*)gc.bq;
  g.bs = gc.bs;
  g.M = gc.M;
  g.N = gc.N;
  g.K = gc.K;
  g.ldc = gc.ldc;
  g.tiles_m = (int)tiles_m;
  g.tiles_n = (int)tiles_n;
  if (OUT == OUT_F32) {
    g.c = gc.c;
    g.cs = nullptr;
    g.vec = ((uintptr_t)gc.c % 16) == 0 && gc.ldc % 4 == 0;
  } else if (OUT == OUT_BF16) {
    g.c = gc.out_q;
    g.cs = nullptr;
    g.vec = ((uintptr_t)gc.out_q % 8) == 0 && gc.ldc % 4 == 0;
  } else {
    g.c = gc.out_q;
    g.cs = gc.out_s;
    g.vec = 0;
  }
  // one workgroup per compute unit (a multiple of 8, so that a workgroup's
  // tiles stay on its XCD), or one per tile when there are fewer tiles
  const int64_t T = tiles_m * tiles_n;
  int64_t G = device_cus() & ~7;
  if (G < 8) G = 8;
  if (T < G) G = T;
  // XCD blocks where the tile grid splits evenly into 8 blocks of at least G / 8
  // tiles: the split whose blocks need the fewest panel bytes
  g.part_m = g.part_n = 0;
  if (G % 8 == 0 && T >= G) {
    int64_t best = -1;
    for (int pm = 1; pm <= 8; pm *= 2) {
      const int pn = 8 / pm;
      if (tiles_m % pm || tiles_n % pn || (tiles_m / pm) * (tiles_n / pn) < G / 8) continue;
      const int64_t bytes = (tiles_m / pm) * (gc.K * Fmt<FA>::bits / 8) + (tiles_n / pn) * (gc.K * Fmt<FB>::bits / 8);
      if (best < 0 || bytes < best) {
        best = bytes;
        g.part_m = pm;
        g.part_n = pn;
      }
    }
  }
  hipLaunchKernelGGL((k_gemm_fast<FA, FB, KS, OUT, SPREAD>), dim3((unsigned)G), dim3(256), 0, gc.st, g);
  return hipGetLastError();
}

// fp32 and bf16 output spread each scale chunk's loads over its stages where
// every chunk is whole and a tile has at least two (K % 1024 == 0, K >= 2048)
template <int FA, int FB, int KS>
static hipError_t launch_fast_out(const GemmCall& gc, int64_t tiles_m, int64_t tiles_n) {
  const bool spread = gc.K % 1024 == 0 && gc.K >= 2048;
  if (gc.out_fmt == GEMM_OUT_BF16)
    return spread ? launch_fast<FA, FB, KS, OUT_BF16, true>(gc, tiles_m, tiles_n)
                  : launch_fast<FA, FB, KS, OUT_BF16>(gc, tiles_m, tiles_n);
  if (gc.out_fmt < 0)
    return spread ? launch_fast<FA, FB, KS, OUT_F32, true>(gc, tiles_m, tiles_n)
                  : launch_fast<FA, FB, KS, OUT_F32>(gc, tiles_m, tiles_n);
  if constexpr (FA == INT8) {  // MXINT8 products leave as fp32 or bf16 only
    return hipErrorNotSupported;
  } else {
    switch (gc.out_fmt) {
      case E4M3: return launch_fast<FA, FB, KS, OUT_MX_E4M3>(gc, tiles_m, tiles_n);
      case E5M2: return launch_fast<FA, FB, KS, OUT_MX_E5M2>(gc, tiles_m, tiles_n);
      case E2M1: return launch_fast<FA, FB, KS, OUT_MX_E2M1>(gc, tiles_m, tiles_n);
      default: return hipErrorNotSupported;
    }
  }
}

template <int FA, int FB>
hipError_t gemm_launch(const GemmCall& gc) {
  const int64_t M = gc.M, N = gc.N, K = gc.K;
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  // The staged kernel addresses operands and scales with 32-bit buffer
  // offsets (rows rounded up to whole tiles, plus the reach of the last chunk,
  // stay below 2^32 bytes) and loads scale rows 16 bytes at a time.
  const int64_t lim = (int64_t)1 << 32;
  const int64_t nblk = K / 32;
  const bool fast = K > 0 && K % 512 == 0 && ((uintptr_t)gc.as % 16) == 0 &&
                    ((uintptr_t)gc.bs % 16) == 0 &&
                    tiles_m * BM * (K * Fmt<FA>::bits / 8) + K < lim &&
                    tiles_n * BN * (K * Fmt<FB>::bits / 8) + K < lim &&
                    tiles_m * BM * nblk + 64 < lim && tiles_n * BN * nblk + 64 < lim &&
                    tiles_m * tiles_n < ((int64_t)1 << 31);
  if (fast) {
    if constexpr (Fmt<FA>::bits == 4 && Fmt<FB>::bits == 4)
      return launch_fast_out<FA, FB, 256>(gc, tiles_m, tiles_n);
    else
      return launch_fast_out<FA, FB, 128>(gc, tiles_m, tiles_n);
  }
  if (gc.out_fmt >= 0 && gc.out_fmt != GEMM_OUT_BF16) return hipErrorNotSupported;  // MX output: staged only
  if constexpr (FA == INT8) {
    return gemm_i8_launch<FA>(gc.aq, gc.as, gc.bq, gc.bs, M, N, K, gc.c, gc.ldc, gc.out_fmt, gc.out_q,
                              gc.st);
  } else {
    if (gc.out_fmt == GEMM_OUT_BF16)
      hipLaunchKernelGGL((k_gemm<FA, FB, true>), dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0,
                         gc.st, (const uint8_t*)gc.aq, gc.as, (const uint8_t*)gc.bq, gc.bs, M, N, K,
                         gc.c, (uint16_t*)gc.out_q, gc.ldc, (int)tiles_n);
    else
      hipLaunchKernelGGL((k_gemm<FA, FB, false>), dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0,
                         gc.st, (const uint8_t*)gc.aq, gc.as, (const uint8_t*)gc.bq, gc.bs, M, N, K,
                         gc.c, nullptr, gc.ldc, (int)tiles_n);
    return hipGetLastError();
  }
}

}  // namespace mx
