/*
 * mx_oracle.h -- CPU reference of Microscaling (MX) block quantization and of the
 * block-scaled dot product.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant with the GPU library; the two agree only because
 * both follow the same definitions:
 *
 *   "Microscaling Data Formats for Deep Learning" (Rouhani et al., arXiv
 *   2310.10537), source-linked summary page:
 *     Section 2 "Microscaling"      -- an MX block is one shared scale X plus k
 *                                      narrow elements P_i; value v_i = X * P_i;
 *                                      a NaN scale makes the whole block NaN;
 *                                      the scale is E8M0.
 *     Section 3 "Scalar Float to MX Format Conversion" (Algorithm 1) -- the
 *                                      shared exponent is the largest input
 *                                      exponent less the element format's
 *                                      largest exponent; each P_i quantizes
 *                                      V_i / X with overflowing normals clamped;
 *                                      subnormal fp32 inputs become zero; the
 *                                      scale axis matters (no commuting with a
 *                                      transpose).
 *     Section 4 "Compute Flow"      -- dot products take MX inputs and return
 *                                      scalar floats.
 *   "Format-Aware Fusion for Fast FP4 Pretraining" (arXiv abstract page) --
 *                                      MXFP4 with stochastic rounding of
 *                                      row-gradient operands and a fixed-sign
 *                                      32-value Hadamard transform.
 *
 * Element-format parameters (bias, largest exponent, max normal, NaN codes) are
 * those of the public OCP MX v1.0 / OCP 8-bit floating point definitions; the
 * pages name the formats but do not print them.
 *
 * Partial blocks: the pages define blocks of k elements and leave the storage
 * to the implementation.  A blocked dimension n that is not a multiple of 32
 * is taken as the tensor extended with zeros to n_p = 32 * ceil(n / 32): the
 * packed outputs hold n_p elements per row (padded positions included) and
 * n_p / 32 scales, the logical index of an element for stochastic rounding is
 * row * C_p + col with C_p = 32 * ceil(cols / 32), and a dot product runs over
 * the padded length.  For n % 32 == 0 nothing changes.
 *
 * Every pointer here is a HOST pointer.  Byte arrays hold packed element codes
 * exactly as the GPU library stores them (FP8/INT8: one byte per element;
 * FP6: 24 bytes per 32-element block, element j in bits 6j..6j+5 of the
 * little-endian 192-bit block; FP4: two elements per byte, even index in the
 * low nibble).  Scales are one E8M0 byte per block.
 */
#ifndef MX_ORACLE_H
#define MX_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element formats (same numbering as the public library's enum) */
enum { MXO_E4M3 = 0, MXO_E5M2 = 1, MXO_E2M3 = 2, MXO_E3M2 = 3, MXO_E2M1 = 4, MXO_INT8 = 5 };
enum { MXO_SRC_F32 = 0, MXO_SRC_BF16 = 1 };
enum { MXO_RNE = 0, MXO_SR = 1 };
enum { MXO_LAYOUT_ROW = 1, MXO_LAYOUT_COLT = 2 };
enum { MXO_FLAG_HADAMARD32 = 1 };

/* Decoded value of one element code (NaN / Inf where the format has them). */
double mxo_elem_value(int fmt, unsigned code);
/* Format parameters: largest normal exponent, max normal magnitude, element bits. */
int mxo_elem_emax(int fmt);
double mxo_elem_maxnorm(int fmt);
int mxo_elem_bits(int fmt);

/* Quantize one 32-element block (Algorithm 1).  `rnd` holds one 32-bit random
 * word per element for stochastic rounding and may be NULL for RNE.  Writes 32
 * unpacked element codes and the E8M0 scale code. */
void mxo_quantize_block(int fmt, const float v[32], int round, const uint32_t* rnd,
                        uint8_t codes[32], uint8_t* scale);

/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): one block of 4 words. */
void mxo_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* The 32-bit random word stochastic rounding uses for the element with logical
 * source index i (row * cols + col) in the given layout (0 row-wise, 1
 * column-wise). */
uint32_t mxo_sr_word(uint64_t seed, uint64_t counter_offset, int layout_id, uint64_t i);

/* Fixed-sign 32-point Hadamard transform in fp32, in place. */
void mxo_hadamard32(float x[32], uint32_t signs);

/* Packed bytes for a [rows x cols] element array whose blocks run along cols
 * (cols padded to a multiple of 32). */
int64_t mxo_packed_bytes(int fmt, int64_t rows, int64_t cols);

/* Whole-tensor quantize.  x is [rows x cols] with leading dimension ld (in
 * elements), fp32 or bf16 bit patterns.  With R_p, C_p the dimensions padded
 * to multiples of 32: row-wise outputs q_row [rows x C_p] packed, s_row
 * [rows x C_p/32]; column-wise outputs stored transposed, q_colt [cols x R_p]
 * packed, s_colt [cols x R_p/32].  Returns 0 on success, -1 on a bad
 * argument. */
int mxo_quantize(int src, const void* x, int64_t rows, int64_t cols, int64_t ld,
                 int fmt, unsigned layouts, int round, unsigned flags,
                 uint64_t seed, uint64_t counter_offset, uint32_t hadamard_signs,
                 uint8_t* q_row, uint8_t* s_row, uint8_t* q_colt, uint8_t* s_colt);

/* Dequantize a packed [rows x C_p] tensor whose blocks run along cols to fp32
 * y [rows x cols] (the padded positions are dropped). */
int mxo_dequantize(const uint8_t* q, const uint8_t* s, int fmt, int64_t rows, int64_t cols,
                   float* y);

/* C[m,n] = sum_k a[m,k] * b[n,k] over the dequantized operands, in fp64, with
 * T[m,n] = sum_k |a[m,k] * b[n,k]|.  A is [M x K], B is given as B^T [N x K];
 * both have their blocks along K, and k runs over K padded to a multiple of
 * 32 (the padded positions are part of the operands).  t may be NULL. */
int mxo_gemm_f64(const uint8_t* a_q, const uint8_t* a_s, int a_fmt,
                 const uint8_t* b_q, const uint8_t* b_s, int b_fmt,
                 int64_t M, int64_t N, int64_t K, double* c, double* t);

/* The same dot products for `count` selected (m, n) pairs only. */
int mxo_gemm_f64_at(const uint8_t* a_q, const uint8_t* a_s, int a_fmt,
                    const uint8_t* b_q, const uint8_t* b_s, int b_fmt,
                    int64_t M, int64_t N, int64_t K,
                    const int64_t* ms, const int64_t* ns, int64_t count,
                    double* c, double* t);

/* Threads of the whole-tensor functions (n <= 0 leaves them unchanged);
 * returns the number in force. */
int mxo_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
