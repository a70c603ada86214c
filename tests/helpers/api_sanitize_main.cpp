// Host-only driver of the C-ABI validation layer (mx_api.cpp), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py.
// The kernel launchers are replaced by stubs that record the call and check
// the arguments validation hands them, so every entry point runs to its end
// on the host without a GPU.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "mx.h"
#include "mx_internal.h"

namespace mx {
static int calls = 0;
static QuantArgs last_q;
hipError_t launch_quant_rows(const QuantArgs& a, hipStream_t) {
  calls++;
  last_q = a;
  return hipSuccess;
}
hipError_t launch_quant_tiles(const QuantArgs& a, bool, hipStream_t) {
  calls++;
  last_q = a;
  return hipSuccess;
}
hipError_t launch_dequant(const void*, const uint8_t*, int, int64_t, int64_t, float*, hipStream_t) {
  calls++;
  return hipSuccess;
}
static int64_t last_k = -1;
hipError_t launch_gemm(const void*, const uint8_t*, int, const void*, const uint8_t*, int, int64_t,
                       int64_t, int64_t K, float*, int64_t, int, uint8_t*, uint8_t*, hipStream_t) {
  calls++;
  last_k = K;
  return hipSuccess;
}
}  // namespace mx

static int fails = 0;
#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #cond); \
      fails++;                                                   \
    }                                                            \
  } while (0)

int main() {
  // real host buffers stand in for device pointers: the layer never touches them
  alignas(16) static uint8_t buf[1 << 16];
  void* P = buf;
  mx_quant_params p;
  std::memset(&p, 0, sizeof p);
  p.src = MX_SRC_BF16;
  p.fmt = MX_E4M3;
  p.layouts = MX_LAYOUT_ROW;
  // every format, layout, rounding and source, whole and partial blocks
  for (int fmt = 0; fmt < 6; fmt++)
    for (unsigned lay = 1; lay <= 3; lay++)
      for (int src = 0; src < 2; src++)
        for (int64_t cols : {1, 31, 32, 70, 4096})
          for (int64_t rows : {1, 33, 64}) {
            p.fmt = fmt;
            p.layouts = lay;
            p.src = src;
            p.round = (int)(cols & 1);
            const int64_t ld = (cols + 7) / 8 * 8;
            const int before = mx::calls;
            CHECK(mx_quantize(P, rows, cols, ld, &p, P, buf, P, buf, nullptr) == MX_OK);
            CHECK(mx::calls == before + 1);
            CHECK(mx::last_q.rows == rows && mx::last_q.cols == cols);
          }
  p.fmt = MX_E4M3;
  p.layouts = MX_LAYOUT_ROW;
  p.src = MX_SRC_BF16;
  p.round = MX_RNE;
  CHECK(mx_quantize(P, 4, 64, 64, nullptr, P, buf, P, buf, nullptr) == MX_ERR_ARG);
  CHECK(mx_quantize(P, 4, 64, 60, &p, P, buf, P, buf, nullptr) == MX_ERR_SHAPE);
  CHECK(mx_quantize(buf + 4, 4, 64, 64, &p, P, buf, P, buf, nullptr) == MX_ERR_ALIGN);
  CHECK(mx_quantize(P, -1, 64, 64, &p, P, buf, P, buf, nullptr) == MX_ERR_ARG);
  p.fmt = 7;
  CHECK(mx_quantize(P, 4, 64, 64, &p, P, buf, P, buf, nullptr) == MX_ERR_ARG);
  p.fmt = MX_E4M3;
  CHECK(mx_quantize(nullptr, 0, 64, 64, &p, nullptr, nullptr, nullptr, nullptr, nullptr) == MX_OK);
  // dequantize
  for (int fmt = 0; fmt < 6; fmt++)
    for (int64_t cols : {1, 32, 70})
      CHECK(mx_dequantize(P, buf, fmt, 3, cols, (float*)P, nullptr) == MX_OK);
  CHECK(mx_dequantize(P, buf, 9, 3, 32, (float*)P, nullptr) == MX_ERR_ARG);
  CHECK(mx_dequantize(buf + 1, buf, 0, 3, 32, (float*)P, nullptr) == MX_ERR_ALIGN);
  // gemm: K padded to whole blocks on the way to the kernels
  for (int a = 0; a < 6; a++)
    for (int b = 0; b < 6; b++)
      for (int64_t K : {0, 1, 32, 70, 512, 1000}) {
        const int want = ((a == MX_INT8) != (b == MX_INT8)) ? MX_ERR_UNSUPPORTED : MX_OK;
        CHECK(mx_gemm(P, buf, a, P, buf, b, 5, 7, K, (float*)P, 7, nullptr) == want);
        if (want == MX_OK) CHECK(mx::last_k == (K + 31) / 32 * 32);
        CHECK(mx_gemm_bf16(P, buf, a, P, buf, b, 5, 7, K, (uint16_t*)P, 7, nullptr) == want);
      }
  CHECK(mx_gemm(P, buf, 0, P, buf, 0, 5, 7, 64, (float*)P, 6, nullptr) == MX_ERR_SHAPE);
  CHECK(mx_gemm(P, buf, 0, P, buf, 0, 5, 7, 64, nullptr, 7, nullptr) == MX_ERR_ARG);
  for (int cf = 0; cf < 6; cf++) {
    const int want = (cf == MX_E4M3 || cf == MX_E5M2 || cf == MX_E2M1) ? MX_OK : MX_ERR_UNSUPPORTED;
    CHECK(mx_gemm_mx(P, buf, 0, P, buf, 0, 5, 100, 512, cf, P, buf, nullptr) == want);
  }
  // helpers
  for (int fmt = 0; fmt < 6; fmt++)
    for (int64_t cols : {0, 1, 31, 32, 33, 4095}) {
      const int64_t bits = (fmt == 2 || fmt == 3) ? 6 : (fmt == 4 ? 4 : 8);
      CHECK(mx_packed_bytes(fmt, 3, cols) == 3 * ((cols + 31) / 32) * 32 * bits / 8);
      CHECK(mx_scale_bytes(3, cols) == 3 * ((cols + 31) / 32));
    }
  CHECK(mx_packed_bytes(-1, 3, 32) == -1);
  for (int s = -6; s <= 1; s++) CHECK(std::strlen(mx_status_str(s)) > 0);
  CHECK(std::strlen(mx_version()) > 0);
  if (fails) return 1;
  std::printf("api validation: %d launcher calls, all checks passed\n", mx::calls);
  return 0;
}
