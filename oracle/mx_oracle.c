/*
 * mx_oracle.c -- plain, slow CPU reference of MX quantization and the MX dot
 * product.  TEST INFRASTRUCTURE ONLY (see mx_oracle.h): nothing on the product
 * path links or calls this file.
 *
 * Written for obviousness, not speed: every element is quantized by exact
 * fp64 arithmetic on its value (no bit tricks), blocks are visited one by one,
 * and the dot product dequantizes into fp64 and sums term by term.
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes of the repository):
 *   - block size 32; element-format parameters from OCP MX v1.0 / OCP FP8;
 *   - floor(log2(amax)) is taken exactly (frexp), never through a floating log2;
 *   - an all-zero block gets the smallest scale, code 0 (2^-127);
 *   - a block holding Inf or NaN gets the NaN scale 0xFF; its elements are the
 *     format's NaN code (E4M3, E5M2: 0x7F) or 0 where the format has no NaN;
 *   - element rounding is round-to-nearest-even unless stochastic rounding is
 *     asked for; saturation to the largest normal happens after rounding;
 *   - a zero result keeps the input's sign in the FP formats; INT8 has only +0;
 *   - INT8 elements are n/64 with n in [-127, 127];
 *   - stochastic rounding rounds the magnitude up iff r < F, where r is the
 *     element's 32-bit Philox word and F = floor(frac * 2^32) for the discarded
 *     fraction frac of one grid step;
 *   - subnormal fp32 values are flushed to signed zero when loaded and again at
 *     the input of the block conversion (after the optional Hadamard step);
 *   - a blocked dimension that is not a multiple of 32 is padded with zeros to
 *     the next multiple (the pages fix no convention for a short block): the
 *     missing elements of the last block read as +0, the packed row holds the
 *     whole padded block, and stochastic-rounding indices are taken in the
 *     padded tensor.
 */
#include "mx_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Element formats (OCP MX v1.0 / OCP 8-bit FP).                              */
/* ------------------------------------------------------------------------- */
typedef struct {
  int is_int;     /* MXINT8: fixed point n / 64                                */
  int ebits;      /* exponent bits                                             */
  int mbits;      /* mantissa bits                                             */
  int bias;       /* exponent bias                                             */
  int emin;       /* exponent of the smallest normal binade = 1 - bias         */
  int emax;       /* exponent of the largest normal binade                     */
  double maxnorm; /* largest finite magnitude                                  */
  int nan_code;   /* positive NaN code, -1 when the format has no NaN          */
  int bits;       /* storage bits per element                                  */
} fmt_desc;

static const fmt_desc FMTS[6] = {
    /* E4M3: exponent field 15 holds normals except mantissa 111 (NaN), so the
     * top binade is 2^8 and the largest magnitude is 1.75 * 2^8 = 448. */
    {0, 4, 3, 7, -6, 8, 448.0, 0x7F, 8},
    /* E5M2: exponent field 31 is Inf / NaN; top binade 2^15; 1.75 * 2^15. */
    {0, 5, 2, 15, -14, 15, 57344.0, 0x7F, 8},
    /* E2M3: no Inf / NaN; top binade 2^2; 1.875 * 4 = 7.5. */
    {0, 2, 3, 1, 0, 2, 7.5, -1, 6},
    /* E3M2: no Inf / NaN; top binade 2^4; 1.75 * 16 = 28. */
    {0, 3, 2, 3, -2, 4, 28.0, -1, 6},
    /* E2M1: no Inf / NaN; top binade 2^2; 1.5 * 4 = 6. */
    {0, 2, 1, 1, 0, 2, 6.0, -1, 4},
    /* INT8: two's complement n with an implicit 2^-6; emax 0; 127/64. */
    {1, 0, 0, 0, 0, 0, 127.0 / 64.0, -1, 8},
};

static int fmt_ok(int fmt) { return fmt >= 0 && fmt <= 5; }

int mxo_elem_emax(int fmt) { return fmt_ok(fmt) ? FMTS[fmt].emax : 0; }
double mxo_elem_maxnorm(int fmt) { return fmt_ok(fmt) ? FMTS[fmt].maxnorm : NAN; }
int mxo_elem_bits(int fmt) { return fmt_ok(fmt) ? FMTS[fmt].bits : 0; }

double mxo_elem_value(int fmt, unsigned code) {
  if (!fmt_ok(fmt)) return NAN;
  const fmt_desc* f = &FMTS[fmt];
  if (f->is_int) return (double)(int8_t)(uint8_t)code / 64.0;
  unsigned sign = (code >> (f->ebits + f->mbits)) & 1u;
  unsigned e = (code >> f->mbits) & ((1u << f->ebits) - 1u);
  unsigned m = code & ((1u << f->mbits) - 1u);
  double s = sign ? -1.0 : 1.0;
  if (fmt == MXO_E4M3 && e == 15 && m == 7) return NAN;
  if (fmt == MXO_E5M2 && e == 31) return m == 0 ? s * INFINITY : NAN;
  if (e == 0) return s * ldexp((double)m, f->emin - f->mbits); /* subnormal */
  return s * ldexp(1.0 + ldexp((double)m, -f->mbits), (int)e - f->bias);
}

/* floor(log2(a)) for a finite a > 0, exactly. */
static int floor_log2(double a) {
  int e;
  frexp(a, &e); /* a = f * 2^e with f in [0.5, 1) */
  return e - 1;
}

/* Code of the finite magnitude q (already on the format's grid and <= maxnorm),
 * with the sign bit `neg`. */
static uint8_t encode_fp(const fmt_desc* f, int neg, double q) {
  unsigned sign = (unsigned)neg << (f->ebits + f->mbits);
  if (q == 0.0) return (uint8_t)sign;
  if (q < ldexp(1.0, f->emin)) { /* subnormal: exponent field 0 */
    unsigned m = (unsigned)(q / ldexp(1.0, f->emin - f->mbits));
    return (uint8_t)(sign | m);
  }
  int e = floor_log2(q);
  unsigned efield = (unsigned)(e + f->bias);
  unsigned m = (unsigned)((q / ldexp(1.0, e) - 1.0) * ldexp(1.0, f->mbits));
  return (uint8_t)(sign | (efield << f->mbits) | m);
}

/* Whether to round the magnitude n + frac (frac in [0, 1), in grid steps) up. */
static int round_up(double n, double frac, int round, uint32_t r) {
  if (round == MXO_SR) {
    double F = floor(frac * 4294967296.0); /* top 32 bits of the fraction */
    return (double)r < F;
  }
  /* round to nearest, ties to even */
  if (frac > 0.5) return 1;
  if (frac < 0.5) return 0;
  return fmod(n, 2.0) == 1.0;
}

/* quantize_to_element_format(y): y = V_i / X, a finite double. */
static uint8_t quantize_elem(const fmt_desc* f, double y, int round, uint32_t r) {
  int neg = signbit(y) != 0;
  double a = fabs(y);
  if (f->is_int) {
    double step = 1.0 / 64.0;
    double n = floor(a / step), frac = a / step - n;
    if (round_up(n, frac, round, r)) n += 1.0;
    if (n > 127.0) n = 127.0; /* saturate */
    int v = neg ? -(int)n : (int)n;
    return (uint8_t)(int8_t)v;
  }
  /* grid step of a's binade (binades below the smallest normal share the
   * subnormal step) */
  int e = (a == 0.0) ? f->emin : floor_log2(a);
  if (e < f->emin) e = f->emin;
  double step = ldexp(1.0, e - f->mbits);
  double n = floor(a / step), frac = a / step - n;
  if (round_up(n, frac, round, r)) n += 1.0;
  double q = n * step;
  if (q > f->maxnorm) q = f->maxnorm; /* overflowing normals clamp to max normal */
  return encode_fp(f, neg, q);
}

static int is_subnormal32(float v) {
  uint32_t b;
  memcpy(&b, &v, 4);
  return ((b >> 23) & 0xFFu) == 0 && (b & 0x7FFFFFu) != 0;
}

static float flush_subnormal(float v) { return is_subnormal32(v) ? copysignf(0.0f, v) : v; }

void mxo_quantize_block(int fmt, const float in[32], int round, const uint32_t* rnd,
                        uint8_t codes[32], uint8_t* scale) {
  const fmt_desc* f = &FMTS[fmt];
  float v[32];
  /* subnormal fp32 inputs become (signed) zero */
  for (int i = 0; i < 32; i++) v[i] = flush_subnormal(in[i]);

  /* Inf or NaN anywhere: the shared scale is not representable -> NaN scale */
  for (int i = 0; i < 32; i++) {
    if (!isfinite(v[i])) {
      *scale = 0xFF;
      for (int j = 0; j < 32; j++) codes[j] = (uint8_t)(f->nan_code >= 0 ? f->nan_code : 0);
      return;
    }
  }

  double amax = 0.0;
  for (int i = 0; i < 32; i++)
    if (fabs((double)v[i]) > amax) amax = fabs((double)v[i]);

  /* shared_exp = floor(log2(amax)) - emax_elem, clamped to E8M0's range */
  int shared_exp = (amax == 0.0) ? -127 : floor_log2(amax) - f->emax;
  if (shared_exp < -127) shared_exp = -127;
  if (shared_exp > 127) shared_exp = 127;
  *scale = (uint8_t)(shared_exp + 127);
  double X = ldexp(1.0, shared_exp);

  for (int i = 0; i < 32; i++) {
    double y = (double)v[i] / X; /* exact: X is a power of two */
    codes[i] = quantize_elem(f, y, round, rnd ? rnd[i] : 0u);
  }
}

/* ------------------------------------------------------------------------- */
/* Philox4x32-10.                                                             */
/* ------------------------------------------------------------------------- */
void mxo_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u; /* round multipliers */
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u; /* Weyl key increments */
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; round++) {
    if (round > 0) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t p0 = (uint64_t)M0 * x0, p1 = (uint64_t)M1 * x2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t y0 = hi1 ^ x1 ^ k0, y1 = lo1, y2 = hi0 ^ x3 ^ k1, y3 = lo0;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

uint32_t mxo_sr_word(uint64_t seed, uint64_t counter_offset, int layout_id, uint64_t i) {
  uint64_t j = counter_offset + (i >> 2);
  uint32_t ctr[4] = {(uint32_t)j, (uint32_t)(j >> 32), (uint32_t)layout_id, 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  mxo_philox4x32_10(ctr, key, out);
  return out[i & 3];
}

/* ------------------------------------------------------------------------- */
/* Fixed-sign Hadamard-32 in fp32.                                            */
/* ------------------------------------------------------------------------- */
void mxo_hadamard32(float x[32], uint32_t signs) {
  for (int j = 0; j < 32; j++)
    if ((signs >> j) & 1u) x[j] = -x[j];
  for (int h = 1; h < 32; h <<= 1) {
    for (int j = 0; j < 32; j++) {
      if (j & h) continue;
      float a = x[j], b = x[j + h];
      x[j] = a + b;
      x[j + h] = a - b;
    }
  }
  const uint32_t c_bits = 0x3E3504F3u; /* 1/sqrt(32) rounded to nearest fp32 */
  float c;
  memcpy(&c, &c_bits, 4);
  for (int j = 0; j < 32; j++) x[j] = x[j] * c;
}

/* ------------------------------------------------------------------------- */
/* Packing.                                                                   */
/* ------------------------------------------------------------------------- */
/* n rounded up to whole 32-element blocks */
static int64_t padded(int64_t n) { return (n + 31) / 32 * 32; }

int64_t mxo_packed_bytes(int fmt, int64_t rows, int64_t cols) {
  if (!fmt_ok(fmt) || rows < 0 || cols < 0) return -1;
  return rows * (padded(cols) * FMTS[fmt].bits / 8);
}

/* bytes of one packed row of `cols` elements (a whole number of blocks) */
static int64_t row_bytes(int fmt, int64_t cols) { return padded(cols) * FMTS[fmt].bits / 8; }

static void put_code(uint8_t* row, int fmt, int64_t j, uint8_t code) {
  int bits = FMTS[fmt].bits;
  if (bits == 8) {
    row[j] = code;
  } else if (bits == 4) {
    uint8_t* p = &row[j >> 1];
    if (j & 1) *p = (uint8_t)((*p & 0x0F) | ((code & 0xF) << 4));
    else *p = (uint8_t)((*p & 0xF0) | (code & 0xF));
  } else { /* 6 bits, 24 bytes per block, little-endian bit order */
    uint8_t* blk = row + (j / 32) * 24;
    int bit = (int)(j % 32) * 6;
    for (int b = 0; b < 6; b++, bit++) {
      uint8_t mask = (uint8_t)(1u << (bit & 7));
      if ((code >> b) & 1u) blk[bit >> 3] |= mask;
      else blk[bit >> 3] &= (uint8_t)~mask;
    }
  }
}

static unsigned get_code(const uint8_t* row, int fmt, int64_t j) {
  int bits = FMTS[fmt].bits;
  if (bits == 8) return row[j];
  if (bits == 4) return (j & 1) ? (row[j >> 1] >> 4) : (row[j >> 1] & 0xF);
  const uint8_t* blk = row + (j / 32) * 24;
  int bit = (int)(j % 32) * 6;
  unsigned c = 0;
  for (int b = 0; b < 6; b++, bit++) c |= (unsigned)((blk[bit >> 3] >> (bit & 7)) & 1u) << b;
  return c;
}

/* ------------------------------------------------------------------------- */
/* Whole tensors.                                                             */
/* ------------------------------------------------------------------------- */
static float load_elem(int src, const void* x, int64_t idx) {
  if (src == MXO_SRC_F32) return ((const float*)x)[idx];
  uint32_t b = (uint32_t)((const uint16_t*)x)[idx] << 16; /* bf16 widens exactly */
  float v;
  memcpy(&v, &b, 4);
  return v;
}

/* One block: 32 source elements (strided), of which the first `valid` exist
 * and the rest are the zero padding of a short last block; optional Hadamard,
 * Algorithm 1. */
static void quantize_one(int src, const void* x, int64_t base, int64_t stride, int valid, int fmt,
                         int round, unsigned flags, uint64_t seed, uint64_t off, uint32_t signs,
                         int layout_id, int64_t logical0, int64_t logical_stride, uint8_t codes[32],
                         uint8_t* scale) {
  float v[32];
  uint32_t rnd[32];
  for (int k = 0; k < 32; k++)
    v[k] = k < valid ? flush_subnormal(load_elem(src, x, base + k * stride)) : 0.0f;
  if (flags & MXO_FLAG_HADAMARD32) mxo_hadamard32(v, signs);
  if (round == MXO_SR)
    for (int k = 0; k < 32; k++)
      rnd[k] = mxo_sr_word(seed, off, layout_id, (uint64_t)(logical0 + k * logical_stride));
  mxo_quantize_block(fmt, v, round, round == MXO_SR ? rnd : NULL, codes, scale);
}

int mxo_quantize(int src, const void* x, int64_t rows, int64_t cols, int64_t ld, int fmt,
                 unsigned layouts, int round, unsigned flags, uint64_t seed,
                 uint64_t counter_offset, uint32_t hadamard_signs, uint8_t* q_row,
                 uint8_t* s_row, uint8_t* q_colt, uint8_t* s_colt) {
  if (!fmt_ok(fmt) || (src != MXO_SRC_F32 && src != MXO_SRC_BF16)) return -1;
  if (round != MXO_RNE && round != MXO_SR) return -1;
  if (rows < 0 || cols < 0 || ld < cols) return -1;
  if ((layouts & ~3u) || layouts == 0) return -1;

  /* logical (stochastic-rounding) index of element (r, c): r * cp + c in the
   * zero-padded tensor */
  const int64_t cp = padded(cols);
  if (layouts & MXO_LAYOUT_ROW) {
    if (!q_row || !s_row) return -1;
    int64_t nb = cp / 32, rb = row_bytes(fmt, cols);
    memset(q_row, 0, (size_t)(rows * rb));
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
      for (int64_t b = 0; b < nb; b++) {
        uint8_t codes[32], sc;
        const int valid = (int)(cols - b * 32 < 32 ? cols - b * 32 : 32);
        quantize_one(src, x, r * ld + b * 32, 1, valid, fmt, round, flags, seed, counter_offset,
                     hadamard_signs, 0, r * cp + b * 32, 1, codes, &sc);
        s_row[r * nb + b] = sc;
        for (int k = 0; k < 32; k++) put_code(q_row + r * rb, fmt, b * 32 + k, codes[k]);
      }
    }
  }
  if (layouts & MXO_LAYOUT_COLT) {
    if (!q_colt || !s_colt) return -1;
    int64_t nb = padded(rows) / 32, rb = row_bytes(fmt, rows);
    memset(q_colt, 0, (size_t)(cols * rb));
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; c++) {
      for (int64_t b = 0; b < nb; b++) {
        uint8_t codes[32], sc;
        const int valid = (int)(rows - b * 32 < 32 ? rows - b * 32 : 32);
        quantize_one(src, x, b * 32 * ld + c, ld, valid, fmt, round, flags, seed, counter_offset,
                     hadamard_signs, 1, b * 32 * cp + c, cp, codes, &sc);
        s_colt[c * nb + b] = sc;
        for (int k = 0; k < 32; k++) put_code(q_colt + c * rb, fmt, b * 32 + k, codes[k]);
      }
    }
  }
  return 0;
}

/* value of element (r, j) of a packed tensor of `cols` elements per row
 * (blocks along the row, padded), with its block scale, in fp64 */
static double deq_elem(const uint8_t* q, const uint8_t* s, int fmt, int64_t cols, int64_t r,
                       int64_t j) {
  uint8_t sc = s[r * (padded(cols) / 32) + j / 32];
  if (sc == 0xFF) return NAN; /* NaN scale: the whole block is NaN */
  double p = mxo_elem_value(fmt, get_code(q + r * row_bytes(fmt, cols), fmt, j));
  return ldexp(p, (int)sc - 127); /* v = X * P, exact in fp64 */
}

int mxo_dequantize(const uint8_t* q, const uint8_t* s, int fmt, int64_t rows, int64_t cols,
                   float* y) {
  if (!fmt_ok(fmt) || rows < 0 || cols < 0) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++)
    for (int64_t j = 0; j < cols; j++)
      y[r * cols + j] = (float)deq_elem(q, s, fmt, cols, r, j); /* overflow -> Inf */
  return 0;
}

/* sum over the whole padded length of K: the padded positions hold whatever
 * the operands' last blocks hold there */
static void dot_f64(const uint8_t* a_q, const uint8_t* a_s, int a_fmt, const uint8_t* b_q,
                    const uint8_t* b_s, int b_fmt, int64_t K, int64_t m, int64_t n, double* c,
                    double* t) {
  double acc = 0.0, abs_acc = 0.0;
  for (int64_t k = 0; k < padded(K); k++) {
    double p = deq_elem(a_q, a_s, a_fmt, K, m, k) * deq_elem(b_q, b_s, b_fmt, K, n, k);
    acc += p;
    abs_acc += fabs(p);
  }
  *c = acc;
  if (t) *t = abs_acc;
}

int mxo_gemm_f64(const uint8_t* a_q, const uint8_t* a_s, int a_fmt, const uint8_t* b_q,
                 const uint8_t* b_s, int b_fmt, int64_t M, int64_t N, int64_t K, double* c,
                 double* t) {
  if (!fmt_ok(a_fmt) || !fmt_ok(b_fmt) || M < 0 || N < 0 || K < 0) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; m++)
    for (int64_t n = 0; n < N; n++)
      dot_f64(a_q, a_s, a_fmt, b_q, b_s, b_fmt, K, m, n, &c[m * N + n], t ? &t[m * N + n] : NULL);
  return 0;
}

int mxo_gemm_f64_at(const uint8_t* a_q, const uint8_t* a_s, int a_fmt, const uint8_t* b_q,
                    const uint8_t* b_s, int b_fmt, int64_t M, int64_t N, int64_t K,
                    const int64_t* ms, const int64_t* ns, int64_t count, double* c, double* t) {
  if (!fmt_ok(a_fmt) || !fmt_ok(b_fmt) || K < 0) return -1;
  for (int64_t i = 0; i < count; i++)
    if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return -1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t i = 0; i < count; i++)
    dot_f64(a_q, a_s, a_fmt, b_q, b_s, b_fmt, K, ms[i], ns[i], &c[i], t ? &t[i] : NULL);
  return 0;
}

/* OpenMP threads the whole-tensor functions use (for timing the oracle on one
 * core and on all of them); returns the count now in force. */
int mxo_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
}
