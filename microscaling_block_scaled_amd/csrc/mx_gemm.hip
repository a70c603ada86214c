// mx_gemm.hip -- block-scaled MX matrix multiply on gfx950's
// V_MFMA_SCALE_F32_16X16X128_F8F6F4.
//
// C[m,n] = sum over 32-element blocks kb of 2^(sa[m,kb]-127) * 2^(sb[n,kb]-127)
//          * sum_{k in kb} P_A[m,k] * P_B[n,k]
// ("Microscaling Data Formats for Deep Learning", summary section 4: dot
// products consume MX operands and return scalar floats; section 2: v = X * P).
// The E8M0 scales are applied inside the matrix instruction, accumulation is
// fp32 and C is fp32.
//
// Tiling: a 256-thread workgroup computes a 256 x 256 tile of C; its four
// waves each own 128 x 128 (8 x 8 instructions of 16 x 16 x 128).  Per K-step
// of 128 elements the A and B panels (256 rows each, with their scale bytes)
// are copied global -> registers -> LDS, double buffered, so the copy of step
// s+1 overlaps the instructions of step s.
//
// Operand lane layouts of the 16x16x128 instruction (lane l, row l % 16, block
// kb = l / 16 of the K-step; the scale operand of lane l is the E8M0 byte of
// that row and block):
//   FP8 (E4M3, E5M2): 32 bytes = K-step bytes [16 kb, 16 kb + 16) followed by
//                     [64 + 16 kb, 64 + 16 kb + 16)
//   FP6 (E2M3, E3M2): the 24 packed bytes of block kb
//   FP4 (E2M1):       the 16 packed bytes of block kb
// Result: lane l holds C rows 4 (l / 16) + v, v = 0..3, column l % 16.
#include "mx_device.hpp"
#include "mx_internal.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

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

template <int FA, int FB>
__global__ __launch_bounds__(256) void k_gemm(const uint8_t* __restrict__ aq,
                                              const uint8_t* __restrict__ as,
                                              const uint8_t* __restrict__ bq,
                                              const uint8_t* __restrict__ bs, int64_t M,
                                              int64_t N, int64_t K, float* __restrict__ c,
                                              int64_t ldc, int tiles_n) {
  using L = GemmLds<FA, FB>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
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
        if (row < M && col < N) c[row * ldc + col] = acc[i][j][v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fast path (K % 128 == 0, scale rows 4-byte aligned): operand panels and scale
// bytes go global -> LDS directly (no register staging), through a ring of NST
// LDS stages, so loads run NST - 1 K-steps ahead of the matrix instructions.
// One barrier per K-step.  Panel rows are stored unpadded with their 16-byte
// chunks XOR-swizzled so that the 16 rows a 16-lane group reads fall on
// distinct LDS banks.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) const void* gbl_ptr_t;

constexpr int LDS_MAX = 160 * 1024;

template <int F>
__device__ __forceinline__ int swz(int r) {
  if (Op<F>::CH == 8) return (r >> 1) & 7;
  if (Op<F>::CH == 4) return (r >> 2) & 3;
  return 0;  // FP6 rows (6 chunks): unswizzled
}

template <int FA, int FB> struct FastLds {
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = 256 * Op<FA>::RB;
  static constexpr int SA_OFF = B_OFF + 256 * Op<FB>::RB;
  static constexpr int SB_OFF = SA_OFF + 1024;
  static constexpr int STAGE = SB_OFF + 1024;
  static constexpr int NST0 = LDS_MAX / STAGE;
  static constexpr int NST = NST0 > 4 ? 4 : NST0;
  static constexpr int TOTAL = NST * STAGE;
  // direct-load instructions one wave issues per K-step
  static constexpr int PER_STEP = Op<FA>::CH + Op<FB>::CH + 2;
};

// One panel of one K-step: 256 rows x RB bytes, 4 waves x CH instructions of
// 64 lanes x 16 bytes.  Lane `lane` of segment I = 4p + wave fills physical
// chunk I * 64 + lane of the panel.  Loads go through a buffer resource whose
// size is the operand's byte count: rows past the matrix edge fall outside it
// and read as zero.  Per lane and p only the 32-bit byte offset of the row
// chunk is kept; the K-step's byte offset rides in the scalar offset.
template <int F> struct PanelSrc {
  uint32_t voff[Op<F>::CH];
};

template <int F>
__device__ __forceinline__ void panel_src(PanelSrc<F>& P, int64_t row0, int64_t rowbytes, int wave,
                                          int lane) {
  using O = Op<F>;
#pragma unroll
  for (int p = 0; p < O::CH; p++) {
    const int L = (p * 4 + wave) * 64 + lane;
    const int r = L / O::CH, pc = L % O::CH;
    const int c = pc ^ swz<F>(r);
    P.voff[p] = (uint32_t)((row0 + r) * rowbytes + 16 * c);
  }
}

typedef int v4i __attribute__((ext_vector_type(4)));

// Raw buffer resource over `bytes` bytes at `p` (gfx9 word 3: 32-bit data),
// held in scalar registers.
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
// (wave-uniform; lane i lands at lds_dst + i * size).  Written as one asm block
// that also sets M0, so the compiler does not model it: every wait on it is
// explicit (wait_vm_barrier) and LDS reads of the filled stage come after the
// asm barrier.  The instruction has no register result.
__device__ __forceinline__ void dma16(v4i rs, uint32_t voff, uint32_t soff, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :
               : "v"(voff), "s"(rs), "s"(lds_dst), "s"(soff)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(v4i rs, uint32_t voff, uint32_t soff, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, %3 offen lds"
               :
               : "v"(voff), "s"(rs), "s"(lds_dst), "s"(soff)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <int F>
__device__ __forceinline__ void issue_panel(uint8_t* panel, v4i rs, const PanelSrc<F>& P,
                                            uint32_t kbyte0, int wave) {
  using O = Op<F>;
  const uint32_t base = lds_addr(panel);
#pragma unroll
  for (int p = 0; p < O::CH; p++)
    dma16(rs, P.voff[p], kbyte0, base + (uint32_t)((p * 4 + wave) * 1024));
}

// Four scale bytes (the K-step's four blocks) of panel row wave * 64 + lane.
__device__ __forceinline__ void issue_scales(uint8_t* sp, v4i rs, uint32_t voff, uint32_t b0,
                                             int wave) {
  dma4(rs, voff, b0, lds_addr(sp) + (uint32_t)(wave * 256));
}

// Operand of one 16-row tile: `lb` is this lane's row start in the panel
// (tile 0), `toff` the tile's byte offset (a constant), c0 / c1 the swizzled
// chunks of the lane's block.
template <int F>
__device__ __forceinline__ v8i read_fast(const uint8_t* lb, int toff, int c0, int c1, int kb) {
  using O = Op<F>;
  const uint8_t* base = lb + toff;
  v8i v = {0, 0, 0, 0, 0, 0, 0, 0};
  if (O::bits == 8) {
    const uint4 a = *(const uint4*)(base + 16 * c0);
    const uint4 b = *(const uint4*)(base + 16 * c1);
    v[0] = (int)a.x; v[1] = (int)a.y; v[2] = (int)a.z; v[3] = (int)a.w;
    v[4] = (int)b.x; v[5] = (int)b.y; v[6] = (int)b.z; v[7] = (int)b.w;
  } else if (O::bits == 4) {
    const uint4 a = *(const uint4*)(base + 16 * c0);
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

// Wait until at most n of this wave's buffer->LDS loads are outstanding, then
// the workgroup barrier.  One asm block with a memory clobber: the compiler
// can neither move LDS reads above it nor add waits of its own.
template <int n>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(n) : "memory");
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

typedef float v16f __attribute__((ext_vector_type(16)));

// Operand of one 32-row tile for the 32x32x64 instruction, half-step u of the
// K-step (K-step elements [64u, 64u + 64)).  Lane l: row l % 32, block
// kb = l / 32 of the half-step.  FP8 lanes hold the 16-byte pieces at K offsets
// 16 kb and 32 + 16 kb of the half-step; FP6 / FP4 lanes hold their block.
template <int F>
__device__ __forceinline__ v8i read32(const uint8_t* lb, int toff, int u, int kb, int sw) {
  using O = Op<F>;
  const uint8_t* base = lb + toff;
  v8i v = {0, 0, 0, 0, 0, 0, 0, 0};
  if (O::bits == 8) {
    const uint4 a = *(const uint4*)(base + 16 * ((4 * u + kb) ^ sw));
    const uint4 b = *(const uint4*)(base + 16 * ((4 * u + 2 + kb) ^ sw));
    v[0] = (int)a.x; v[1] = (int)a.y; v[2] = (int)a.z; v[3] = (int)a.w;
    v[4] = (int)b.x; v[5] = (int)b.y; v[6] = (int)b.z; v[7] = (int)b.w;
  } else if (O::bits == 4) {
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

// One K-step on LDS stage `st`: two half-steps of 4 x 4 instructions
// (32x32x64) per wave, the A operand of tile i + 1 read from LDS while the
// instructions of tile i issue.
template <int FA, int FB>
__device__ __forceinline__ void mma_step(const uint8_t* st, v16f (&acc)[4][4], int arow_off,
                                         int brow_off, int kb, int swa, int swb) {
  using L = FastLds<FA, FB>;
  const uint8_t* la = st + L::A_OFF + arow_off * Op<FA>::RB;
  const uint8_t* lb = st + L::B_OFF + brow_off * Op<FB>::RB;
  const uint8_t* sa = st + L::SA_OFF + arow_off * 4 + kb;
  const uint8_t* sb = st + L::SB_OFF + brow_off * 4 + kb;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    v8i bop[4];
    int bsc[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      bop[j] = read32<FB>(lb, j * 32 * Op<FB>::RB, u, kb, swb);
      bsc[j] = sb[j * 128 + 2 * u];
    }
    v8i aop = read32<FA>(la, 0, u, kb, swa);
    int asc = sa[2 * u];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v8i anx = aop;
      int asx = asc;
      if (i < 3) {
        anx = read32<FA>(la, (i + 1) * 32 * Op<FA>::RB, u, kb, swa);
        asx = sa[(i + 1) * 128 + 2 * u];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; j++)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop[j], acc[i][j], FA, FB,
                                                                    0, asc, 0, bsc[j]);
      __builtin_amdgcn_sched_barrier(0);
      aop = anx;
      asc = asx;
    }
  }
}

template <int FA, int FB>
__global__ __launch_bounds__(256) void k_gemm_fast(const uint8_t* __restrict__ aq,
                                                   const uint8_t* __restrict__ as,
                                                   const uint8_t* __restrict__ bq,
                                                   const uint8_t* __restrict__ bs, int64_t M,
                                                   int64_t N, int64_t K, float* __restrict__ c,
                                                   int64_t ldc, int tiles_m, int tiles_n) {
  using L = FastLds<FA, FB>;
  constexpr int NST = L::NST;
  // the LDS ring: NST stages of STAGE bytes
  __shared__ __attribute__((aligned(1024))) uint8_t ring[L::TOTAL];
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a wave-uniform (scalar) value: LDS destinations become scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t arow = K * Op<FA>::bits / 8, brow = K * Op<FB>::bits / 8;
  const int64_t nblk = K / 32;
  const int nk = (int)(K / KS);

  PanelSrc<FA> pa;
  PanelSrc<FB> pb;
  panel_src<FA>(pa, m0, arow, wave, lane);
  panel_src<FB>(pb, n0, brow, wave, lane);
  const v4i ra = make_rsrc(aq, (uint32_t)(M * arow));
  const v4i rb = make_rsrc(bq, (uint32_t)(N * brow));
  const v4i rsa = make_rsrc(as, (uint32_t)(M * nblk));
  const v4i rsb = make_rsrc(bs, (uint32_t)(N * nblk));
  const uint32_t vsa = (uint32_t)((m0 + wave * 64 + lane) * nblk);
  const uint32_t vsb = (uint32_t)((n0 + wave * 64 + lane) * nblk);
  auto issue_step = [&](uint8_t* st, int s) {
    issue_panel<FA>(st + L::A_OFF, ra, pa, (uint32_t)s * (KS * Op<FA>::bits / 8), wave);
    issue_panel<FB>(st + L::B_OFF, rb, pb, (uint32_t)s * (KS * Op<FB>::bits / 8), wave);
    issue_scales(st + L::SA_OFF, rsa, vsa, (uint32_t)s * 4, wave);
    issue_scales(st + L::SB_OFF, rsb, vsb, (uint32_t)s * 4, wave);
  };
  auto stage = [&](int j) -> uint8_t* { return ring + j * L::STAGE; };

  // per-lane swizzle of the operand rows (rows of different tiles differ by
  // multiples of 32, which leave the swizzle unchanged)
  const int lr32 = lane & 31, kb32 = lane >> 5;
  const int swa = swz<FA>(lr32), swb = swz<FB>(lr32);
  const int arow_off = wm * 128 + lr32, brow_off = wn * 128 + lr32;

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

#pragma unroll
  for (int i = 0; i < NST - 1; i++)
    if (i < nk) issue_step(stage(i), i);

  int cur = 0;  // stage of step s
  for (int s = 0; s < nk; s++) {
    // this wave's loads for step s have landed once at most the loads of the
    // `ahead` later steps already issued are outstanding
    const int ahead = (s + NST - 2 < nk - 1 ? s + NST - 2 : nk - 1) - s;
    if (NST >= 4 && ahead >= 2) wait_vm_barrier<2 * L::PER_STEP>();
    else if (NST >= 3 && ahead >= 1) wait_vm_barrier<L::PER_STEP>();
    else wait_vm_barrier<0>();
    const int nxt = cur == 0 ? NST - 1 : cur - 1;  // stage of step s + NST - 1
    if (s + NST - 1 < nk) issue_step(stage(nxt), s + NST - 1);
    mma_step<FA, FB>(stage(cur), acc, arow_off, brow_off, kb32, swa, swb);
    cur = cur + 1 == NST ? 0 : cur + 1;
  }

  // 32x32 result layout: lane l holds rows 8 (v / 4) + 4 (l / 32) + v % 4,
  // v = 0..15, of column l % 32
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int64_t col = n0 + wn * 128 + j * 32 + lr32;
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const int64_t row = m0 + wm * 128 + i * 32 + 8 * (v >> 2) + 4 * kb32 + (v & 3);
        if (row < M && col < N) c[row * ldc + col] = acc[i][j][v];
      }
    }
  }
}

template <int FA, int FB>
static hipError_t gemm_launch(const void* aq, const uint8_t* as, const void* bq, const uint8_t* bs,
                              int64_t M, int64_t N, int64_t K, float* c, int64_t ldc,
                              hipStream_t st) {
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  // the fast path addresses operands with 32-bit buffer offsets (rows rounded
  // up to whole tiles must stay below 2^32 bytes)
  const int64_t abytes = tiles_m * BM * (K * Op<FA>::bits / 8) + K;
  const int64_t bbytes = tiles_n * BN * (K * Op<FB>::bits / 8) + K;
  const bool fast = K > 0 && K % KS == 0 && ((uintptr_t)as % 4) == 0 && ((uintptr_t)bs % 4) == 0 &&
                    abytes < ((int64_t)1 << 32) && bbytes < ((int64_t)1 << 32);
  if (fast) {
    hipLaunchKernelGGL((k_gemm_fast<FA, FB>), dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, st, (const uint8_t*)aq, as, (const uint8_t*)bq, bs, M, N, K, c,
                       ldc, (int)tiles_m, (int)tiles_n);
    return hipGetLastError();
  }
  using L = GemmLds<FA, FB>;
  static bool attr_done = false;  // benign race: the call is idempotent
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm<FA, FB>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, L::TOTAL);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL((k_gemm<FA, FB>), dim3((unsigned)(tiles_m * tiles_n)), dim3(256), L::TOTAL, st,
                     (const uint8_t*)aq, as, (const uint8_t*)bq, bs, M, N, K, c, ldc,
                     (int)tiles_n);
  return hipGetLastError();
}

hipError_t launch_gemm(const void* aq, const uint8_t* as, int fa, const void* bq,
                       const uint8_t* bs, int fb, int64_t M, int64_t N, int64_t K, float* c,
                       int64_t ldc, hipStream_t st) {
#define MX_G(A, B) \
  if (fa == A && fb == B) return gemm_launch<A, B>(aq, as, bq, bs, M, N, K, c, ldc, st);
#define MX_GA(A) MX_G(A, E4M3) MX_G(A, E5M2) MX_G(A, E2M3) MX_G(A, E3M2) MX_G(A, E2M1)
  MX_GA(E4M3) MX_GA(E5M2) MX_GA(E2M3) MX_GA(E3M2) MX_GA(E2M1)
#undef MX_GA
#undef MX_G
  return hipErrorInvalidValue;
}

}  // namespace mx
