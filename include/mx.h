/*
 * mx.h -- Microscaling (MX) block quantization and block-scaled matrix multiply
 * on AMD Instinct MI355X (gfx950).
 *
 * Definitions followed ("Microscaling Data Formats for Deep Learning",
 * Rouhani et al., arXiv 2310.10537, source-linked summary page):
 *   section 2 "Microscaling": an MX block encodes k values as one shared scale X
 *     and k narrow elements P_i, value v_i = X * P_i; the scale is E8M0; a NaN
 *     scale makes the whole block NaN; the storage layout is left to the
 *     implementation.
 *   section 3 "Scalar Float to MX Format Conversion" (Algorithm 1): X is the power
 *     of two 2^(floor(log2(max|V_i|)) - emax_elem); P_i is V_i / X quantized to the
 *     element format, overflowing normals clamped to the largest normal; subnormal
 *     fp32 inputs are set to zero; the scale axis is the caller's choice, since
 *     conversion and transposition do not commute.
 *   section 4 "Compute Flow": dot products take MX inputs and return scalar
 *     floats.
 * and the "Format-Aware Fusion for Fast FP4 Pretraining" abstract: MXFP4 with
 * stochastic rounding of row-gradient operands and a fixed-sign 32-value Hadamard
 * transform applied before quantization.
 *
 * Block size is 32 elements.  Element formats follow OCP MX v1.0 / OCP FP8.
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers, owned by the caller.  The library
 *     never allocates or frees memory.  Its only global state is the compute-
 *     unit count of each device (which sizes the GEMM's persistent grid),
 *     looked up on first use and kept in a relaxed atomic per device: calls
 *     are thread-safe.  Calls run on the current HIP device.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  Device faults surface at the caller's next
 *     synchronization on that stream.
 *   - Arguments are validated on the host before anything is launched; a
 *     failed check returns a negative mx_status and launches nothing.  A launch
 *     failure returns MX_ERR_HIP.  No C++ exception crosses this interface.
 *   - Empty tensors (a zero dimension) are valid and launch nothing.
 *
 * Storage layouts (the pages leave them to the implementation):
 *   - elements: FP8 and INT8 one byte each; FP6 (E2M3, E3M2) 24 bytes per
 *     32-element block, element j in bits 6j..6j+5 of the little-endian 192-bit
 *     block; FP4 (E2M1) two per byte, even element in the low nibble.
 *   - scales: one E8M0 byte per block, in a separate array.
 *   - partial blocks: a blocked dimension n that is not a multiple of 32 is
 *     stored as if the source were padded with zeros to n_p = 32 * ceil(n/32);
 *     the padded elements of the last block are part of the packed output.
 *   - row-wise layout: blocks run along the columns of the [rows x cols] source;
 *     q_row is [rows x cols_p] packed (row pitch mx_packed_bytes(fmt, 1, cols)),
 *     s_row is [rows x cols_p/32].
 *   - column-wise layout, stored transposed: blocks run along the rows of the
 *     source; q_colt is [cols x rows_p] packed, s_colt is [cols x rows_p/32].
 */
#ifndef MX_H
#define MX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t. */
typedef struct ihipStream_t* mx_stream_t;

typedef enum {
  MX_OK = 0,
  MX_ERR_ARG = -1,         /* bad enum value, null pointer or negative size */
  MX_ERR_SHAPE = -2,       /* leading dimension smaller than the row          */
  MX_ERR_ALIGN = -3,       /* pointer or leading dimension breaks the 16-byte rule */
  MX_ERR_UNSUPPORTED = -4, /* valid request this build does not implement */
  MX_ERR_HIP = -5          /* the HIP runtime refused a launch */
} mx_status;

/* Element formats; the named MX variants are MXFP8 (E4M3, E5M2), MXFP6 (E2M3,
 * E3M2), MXFP4 (E2M1) and MXINT8. */
typedef enum { MX_E4M3 = 0, MX_E5M2 = 1, MX_E2M3 = 2, MX_E3M2 = 3, MX_E2M1 = 4, MX_INT8 = 5 } mx_elem;
typedef enum { MX_SRC_F32 = 0, MX_SRC_BF16 = 1 } mx_src;
typedef enum { MX_RNE = 0, MX_SR = 1 } mx_round;
enum { MX_LAYOUT_ROW = 1u, MX_LAYOUT_COLT = 2u }; /* bitmask; both = one fused pass */
enum { MX_FLAG_HADAMARD32 = 1u };

typedef struct {
  int32_t src;             /* mx_src: fp32 or bf16 source values                       */
  int32_t fmt;             /* mx_elem: element format                                  */
  uint32_t layouts;        /* MX_LAYOUT_ROW, MX_LAYOUT_COLT or both                    */
  int32_t round;           /* mx_round                                                 */
  uint32_t flags;          /* MX_FLAG_HADAMARD32: transform each block before scaling  */
  uint32_t hadamard_signs; /* bit j set: element j of a block is negated before H32    */
  uint64_t seed;           /* stochastic rounding: Philox4x32-10 key                   */
  uint64_t counter_offset; /* stochastic rounding: Philox counter base                 */
} mx_quant_params;

/*
 * mx_quantize -- Algorithm 1 over every 32-element block of a [rows x cols]
 * source (section 3 of the MX summary), in one pass over the source.
 *
 *   x       [rows x cols] fp32 or bf16 (p->src), leading dimension ld_x elements;
 *           16-byte aligned, ld_x * element size a multiple of 16.
 *   p       host pointer to the parameters above.
 *   q_row, s_row    outputs of the row-wise layout (required iff requested).
 *   q_colt, s_colt  outputs of the column-wise layout, transposed (required iff
 *                   requested).  Packed outputs must be 16-byte aligned.
 * Shapes: any rows, cols >= 0; a short last block along the block axis reads
 * the missing elements as +0 (the source is never read past cols).
 *
 * Per block: subnormal fp32 values become signed zero; with MX_FLAG_HADAMARD32
 * the 32 values (along the block axis) are sign-flipped per hadamard_signs,
 * passed through five fp32 butterfly stages (strides 1, 2, 4, 8, 16) and
 * multiplied by fp32 1/sqrt(32), then flushed again; a block holding Inf or NaN
 * gets scale 0xFF and NaN (FP8) or zero elements; an all-zero block gets scale
 * 0; otherwise the scale is floor(log2 amax) - emax + 127 (at least 0) and each
 * element is rounded to nearest even (MX_RNE), or rounded up in magnitude iff
 * r < floor(frac * 2^32) (MX_SR) with r the element's Philox4x32-10 word: key =
 * seed, counter = (j lo, j hi, layout, 0) with j = counter_offset + (i >> 2),
 * i = row * cols + col its source index, word i & 3, layout 0 row-wise and 1
 * column-wise; with a short last block, i is the index in the zero-padded
 * source, row * cols_p + col.  Results saturate at the largest normal; zeros
 * keep their sign except in INT8, whose elements are n/64 with n in
 * [-127, 127].
 */
int mx_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld_x, const mx_quant_params* p,
                void* q_row, uint8_t* s_row, void* q_colt, uint8_t* s_colt, mx_stream_t stream);

/*
 * mx_dequantize -- v_i = X * P_i for a packed [rows x cols] tensor whose blocks
 * run along cols (section 2 of the MX summary).  A NaN scale (0xFF) gives a NaN
 * block; element NaN / Inf codes decode to NaN / Inf; products beyond fp32
 * overflow to Inf; fp32 subnormal results are kept.
 *   q  packed elements [rows x cols_p], 16-byte aligned;  s  [rows x cols_p/32]
 *      scales (cols_p: cols padded to a multiple of 32);
 *   y  [rows x cols] fp32 output, 16-byte aligned (the padding is dropped).
 */
int mx_dequantize(const void* q, const uint8_t* s, int32_t fmt, int64_t rows, int64_t cols,
                  float* y, mx_stream_t stream);

/*
 * mx_gemm -- C = A * B over MX operands, fp32 accumulation, fp32 output
 * (section 4 "Compute Flow" of the MX summary): C[m,n] = sum over blocks kb of
 * 2^(sa[m,kb]-127) * 2^(sb[n,kb]-127) * sum_{k in kb} P_A[m,k] * P_B[n,k].
 *   a_q, a_s  A as [M x K] row-wise MX (blocks along K), format a_fmt.
 *   b_q, b_s  B given as B^T, [N x K] row-wise MX (blocks along K): exactly what
 *             mx_quantize produces for a weight W[N x K] row-wise, or for B[K x N]
 *             with MX_LAYOUT_COLT.
 *   c         [M x N] fp32, leading dimension ldc >= N.
 * Formats: E4M3, E5M2, E2M3, E3M2, E2M1 for either operand (any mix), or
 * MX_INT8 for both (INT8 mixed with another format returns
 * MX_ERR_UNSUPPORTED).  MXINT8 products are formed exactly (each element times
 * its scale is exact in bf16, subnormals included) and summed in fp32.  Any
 * K >= 0: with K % 32 != 0 the operands hold K_p = 32 * ceil(K/32) elements
 * per row (the zero-padded last block mx_quantize writes) and the sums run
 * over all K_p.  Operand pointers 16-byte aligned.
 * Accuracy: |C - C_exact| <= 1e-5 * sum|a * b| on every tested workload with
 * K >= 512.  For FP8 and E3M2 operands the block-scaled instruction truncates
 * products within groups of 8 along K, so a product dominated by one or a few
 * blocks (short K, or block scales spread by 2^60) can exceed that bound by a
 * small factor; E2M1, E2M3 and MXINT8 products are exact.
 * The result of a block whose scale is 0xFF is unspecified (the hardware's
 * NaN-scale behaviour); no configuration here produces such scales from finite
 * inputs.
 */
int mx_gemm(const void* a_q, const uint8_t* a_s, int32_t a_fmt, const void* b_q,
            const uint8_t* b_s, int32_t b_fmt, int64_t M, int64_t N, int64_t K, float* c,
            int64_t ldc, mx_stream_t stream);

/*
 * mx_gemm_bf16 -- the product of mx_gemm, each fp32 element rounded to bf16
 * (nearest even; NaN stays NaN, fp32 subnormals give bf16 subnormals) as it
 * leaves the kernel: the 16-bit output a linear layer hands to the next one.
 * Arguments as for mx_gemm except
 *   c  [M x N] bf16 bit patterns, leading dimension ldc >= N elements,
 *      2-byte aligned (16-byte aligned with ldc % 4 == 0 stores 8 bytes at a time).
 */
int mx_gemm_bf16(const void* a_q, const uint8_t* a_s, int32_t a_fmt, const void* b_q,
                 const uint8_t* b_s, int32_t b_fmt, int64_t M, int64_t N, int64_t K, uint16_t* c,
                 int64_t ldc, mx_stream_t stream);

/*
 * mx_gemm_mx -- the product of mx_gemm written straight out in MX format:
 * each fp32 row block C[m, 32 j .. 32 j + 31] is quantized as Algorithm 1 of
 * the MX summary (section 3) does it -- shared scale from the block max,
 * elements rounded to nearest even, saturated -- inside the GEMM's epilogue,
 * the producer-side quantization of "Format-Aware Fusion for Fast FP4
 * Pretraining".  The codes and scales are the ones mx_quantize (row layout,
 * fp32 source, MX_RNE, no transform) gives for the fp32 C that mx_gemm
 * computes; the fp32 C itself is never written.
 *   a_q .. K   as for mx_gemm.
 *   c_fmt      MX_E4M3, MX_E5M2 or MX_E2M1 (others: MX_ERR_UNSUPPORTED).
 *   c_q        [M x N_p] packed codes, row pitch mx_packed_bytes(c_fmt, 1, N),
 *              16-byte aligned (N_p: N padded to a multiple of 32; a short last
 *              block holds zeros past N).
 *   c_s        [M x N_p/32] scales.
 * The fused epilogue lives in the staged MFMA kernel only: it needs K_p a
 * positive multiple of 512, 16-byte aligned scale arrays and operands under
 * 4 GiB; outside that the call returns MX_ERR_UNSUPPORTED and writes nothing.
 * M == 0 or N == 0 writes nothing.
 */
int mx_gemm_mx(const void* a_q, const uint8_t* a_s, int32_t a_fmt, const void* b_q,
               const uint8_t* b_s, int32_t b_fmt, int64_t M, int64_t N, int64_t K,
               int32_t c_fmt, void* c_q, uint8_t* c_s, mx_stream_t stream);

/* Host-only helpers: bytes of a packed [rows x cols] element array (blocks
 * along cols, a short last block padded to 32 elements) and of its scale
 * array; -1 on a bad argument. */
int64_t mx_packed_bytes(int32_t fmt, int64_t rows, int64_t cols);
int64_t mx_scale_bytes(int64_t rows, int64_t cols);
/* Static description of a status code. */
const char* mx_status_str(int status);
/* Library version string. */
const char* mx_version(void);

#ifdef __cplusplus
}
#endif
#endif
