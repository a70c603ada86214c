// mx_api.cpp -- the C-ABI entry points declared in include/mx.h.
//
// Every argument is checked on the host before anything is launched, so the
// checks run (and are tested) without a GPU.  No exception leaves this file.
#include "../../include/mx.h"

#include <hip/hip_runtime.h>

#include "mx_internal.h"

namespace {

bool fmt_ok(int32_t f) { return f >= MX_E4M3 && f <= MX_INT8; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_HIP; }

// blocks of a dimension of n elements (a short last block is padded)
int64_t blocks(int64_t n) { return (n + 31) / 32; }

}  // namespace

extern "C" {

int64_t mx_packed_bytes(int32_t fmt, int64_t rows, int64_t cols) {
  if (!fmt_ok(fmt) || rows < 0 || cols < 0) return -1;
  return rows * blocks(cols) * (4 * mx::elem_bits(fmt));
}

int64_t mx_scale_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return -1;
  return rows * blocks(cols);
}

const char* mx_status_str(int status) {
  switch (status) {
    case MX_OK: return "ok";
    case MX_ERR_ARG: return "invalid argument";
    case MX_ERR_SHAPE: return "invalid shape";
    case MX_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case MX_ERR_UNSUPPORTED: return "unsupported combination";
    case MX_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* mx_version(void) { return "mx-gfx950 0.1.0"; }

int mx_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld_x, const mx_quant_params* p,
                void* q_row, uint8_t* s_row, void* q_colt, uint8_t* s_colt, mx_stream_t stream) {
  if (!p) return MX_ERR_ARG;
  if (p->src != MX_SRC_F32 && p->src != MX_SRC_BF16) return MX_ERR_ARG;
  if (!fmt_ok(p->fmt)) return MX_ERR_ARG;
  if (p->round != MX_RNE && p->round != MX_SR) return MX_ERR_ARG;
  const uint32_t lay = p->layouts;
  if (lay == 0 || (lay & ~(uint32_t)(MX_LAYOUT_ROW | MX_LAYOUT_COLT))) return MX_ERR_ARG;
  if (p->flags & ~(uint32_t)MX_FLAG_HADAMARD32) return MX_ERR_ARG;
  if (rows < 0 || cols < 0) return MX_ERR_ARG;
  if (ld_x < cols) return MX_ERR_SHAPE;
  const bool do_row = lay & MX_LAYOUT_ROW, do_col = lay & MX_LAYOUT_COLT;
  if (rows == 0 || cols == 0) return MX_OK;
  if (do_row && (!q_row || !s_row)) return MX_ERR_ARG;
  if (do_col && (!q_colt || !s_colt)) return MX_ERR_ARG;
  if (!x) return MX_ERR_ARG;
  const int64_t esz = p->src == MX_SRC_F32 ? 4 : 2;
  if (!aligned16(x) || (ld_x * esz) % 16) return MX_ERR_ALIGN;
  if ((do_row && !aligned16(q_row)) || (do_col && !aligned16(q_colt))) return MX_ERR_ALIGN;

  mx::QuantArgs a;
  a.x = x;
  a.rows = rows;
  a.cols = cols;
  a.ld_bytes = ld_x * esz;
  a.src = p->src;
  a.fmt = p->fmt;
  a.round = p->round;
  a.hadamard = (p->flags & MX_FLAG_HADAMARD32) != 0;
  a.signs = p->hadamard_signs;
  a.seed = p->seed;
  a.counter_offset = p->counter_offset;
  a.q_row = (uint8_t*)q_row;
  a.s_row = s_row;
  a.q_colt = (uint8_t*)q_colt;
  a.s_colt = s_colt;
  hipStream_t st = (hipStream_t)stream;
  if (do_col) return hip_status(mx::launch_quant_tiles(a, do_row, st));
  return hip_status(mx::launch_quant_rows(a, st));
}

int mx_dequantize(const void* q, const uint8_t* s, int32_t fmt, int64_t rows, int64_t cols,
                  float* y, mx_stream_t stream) {
  if (!fmt_ok(fmt)) return MX_ERR_ARG;
  if (rows < 0 || cols < 0) return MX_ERR_ARG;
  if (rows == 0 || cols == 0) return MX_OK;
  if (!q || !s || !y) return MX_ERR_ARG;
  if (!aligned16(q) || !aligned16(y)) return MX_ERR_ALIGN;
  return hip_status(mx::launch_dequant(q, s, fmt, rows, cols, y, (hipStream_t)stream));
}

int mx_gemm(const void* a_q, const uint8_t* a_s, int32_t a_fmt, const void* b_q,
            const uint8_t* b_s, int32_t b_fmt, int64_t M, int64_t N, int64_t K, float* c,
            int64_t ldc, mx_stream_t stream) {
  if (!fmt_ok(a_fmt) || !fmt_ok(b_fmt)) return MX_ERR_ARG;
  if ((a_fmt == MX_INT8) != (b_fmt == MX_INT8)) return MX_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0) return MX_ERR_ARG;
  if (ldc < N) return MX_ERR_SHAPE;
  if (M == 0 || N == 0) return MX_OK;
  if (!c) return MX_ERR_ARG;
  if (K > 0 && (!a_q || !a_s || !b_q || !b_s)) return MX_ERR_ARG;
  if (K > 0 && (!aligned16(a_q) || !aligned16(b_q))) return MX_ERR_ALIGN;
  return hip_status(mx::launch_gemm(a_q, a_s, a_fmt, b_q, b_s, b_fmt, M, N, 32 * blocks(K), c, ldc,
                                    -1, nullptr, nullptr, (hipStream_t)stream));
}

int mx_gemm_bf16(const void* a_q, const uint8_t* a_s, int32_t a_fmt, const void* b_q,
                 const uint8_t* b_s, int32_t b_fmt, int64_t M, int64_t N, int64_t K, uint16_t* c,
                 int64_t ldc, mx_stream_t stream) {
  if (!fmt_ok(a_fmt) || !fmt_ok(b_fmt)) return MX_ERR_ARG;
  if ((a_fmt == MX_INT8) != (b_fmt == MX_INT8)) return MX_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0) return MX_ERR_ARG;
  if (ldc < N) return MX_ERR_SHAPE;
  if (M == 0 || N == 0) return MX_OK;
  if (!c) return MX_ERR_ARG;
  if (K > 0 && (!a_q || !a_s || !b_q || !b_s)) return MX_ERR_ARG;
  if (K > 0 && (!aligned16(a_q) || !aligned16(b_q))) return MX_ERR_ALIGN;
  if ((uintptr_t)c % 2) return MX_ERR_ALIGN;
  return hip_status(mx::launch_gemm(a_q, a_s, a_fmt, b_q, b_s, b_fmt, M, N, 32 * blocks(K), nullptr,
                                    ldc, mx::GEMM_OUT_BF16, (uint8_t*)c, nullptr,
                                    (hipStream_t)stream));
}

int mx_gemm_mx(const void* a_q, const uint8_t* a_s, int32_t a_fmt, const void* b_q,
               const uint8_t* b_s, int32_t b_fmt, int64_t M, int64_t N, int64_t K,
               int32_t c_fmt, void* c_q, uint8_t* c_s, mx_stream_t stream) {
  if (!fmt_ok(a_fmt) || !fmt_ok(b_fmt) || !fmt_ok(c_fmt)) return MX_ERR_ARG;
  if (a_fmt == MX_INT8 || b_fmt == MX_INT8) return MX_ERR_UNSUPPORTED;
  if (c_fmt != MX_E4M3 && c_fmt != MX_E5M2 && c_fmt != MX_E2M1) return MX_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0) return MX_ERR_ARG;
  if (M == 0 || N == 0) return MX_OK;
  if (!c_q || !c_s) return MX_ERR_ARG;
  if (!a_q || !a_s || !b_q || !b_s) return MX_ERR_ARG;
  if (!aligned16(a_q) || !aligned16(b_q) || !aligned16(c_q)) return MX_ERR_ALIGN;
  const hipError_t e = mx::launch_gemm(a_q, a_s, a_fmt, b_q, b_s, b_fmt, M, N, 32 * blocks(K),
                                       nullptr, N, c_fmt, (uint8_t*)c_q, c_s, (hipStream_t)stream);
  return e == hipErrorNotSupported ? MX_ERR_UNSUPPORTED : hip_status(e);
}

}  // extern "C"
