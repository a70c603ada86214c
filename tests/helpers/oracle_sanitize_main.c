/* Driver of the CPU oracle built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_sanitizers.py: every entry point
 * on small whole and ragged tensors of every format, layout and rounding mode,
 * with and without the transform, buffers sized exactly as documented (so an
 * access past them is reported). */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mx_oracle.h"

static uint32_t lcg = 12345u;
static float rnd(void) {
  lcg = lcg * 1664525u + 1013904223u;
  return ldexpf((float)(int32_t)lcg / 2147483648.0f, (int)(lcg >> 27) - 16);
}

int main(void) {
  const int64_t shapes[][2] = {{1, 1}, {7, 31}, {33, 65}, {64, 32}, {40, 70}};
  for (size_t si = 0; si < sizeof shapes / sizeof shapes[0]; si++) {
    const int64_t rows = shapes[si][0], cols = shapes[si][1];
    float* x = malloc((size_t)(rows * cols) * sizeof(float));
    uint16_t* xb = malloc((size_t)(rows * cols) * sizeof(uint16_t));
    for (int64_t i = 0; i < rows * cols; i++) {
      x[i] = rnd();
      uint32_t b;
      memcpy(&b, &x[i], 4);
      xb[i] = (uint16_t)(b >> 16);
    }
    x[0] = 1e-40f;
    for (int fmt = 0; fmt < 6; fmt++)
      for (unsigned lay = 1; lay <= 3; lay++)
        for (int round = 0; round < 2; round++)
          for (unsigned flags = 0; flags < 2; flags++)
            for (int src = 0; src < 2; src++) {
              const int64_t rb = mxo_packed_bytes(fmt, 1, cols), cb = mxo_packed_bytes(fmt, 1, rows);
              uint8_t* qr = malloc((size_t)(rows * rb));
              uint8_t* sr = malloc((size_t)(rows * ((cols + 31) / 32)));
              uint8_t* qc = malloc((size_t)(cols * cb));
              uint8_t* sc = malloc((size_t)(cols * ((rows + 31) / 32)));
              if (mxo_quantize(src, src ? (const void*)xb : (const void*)x, rows, cols, cols, fmt, lay,
                               round, flags, 42, 3, 0x1234u, qr, sr, qc, sc) != 0)
                return 1;
              if (lay & 1) {
                float* y = malloc((size_t)(rows * cols) * sizeof(float));
                if (mxo_dequantize(qr, sr, fmt, rows, cols, y) != 0) return 2;
                free(y);
                const int64_t K = cols;
                const int64_t nc = rows * rows > 2 ? rows * rows : 2; /* >= the 2 sampled outputs */
                double* c = malloc((size_t)nc * sizeof(double));
                double* t = malloc((size_t)nc * sizeof(double));
                if (mxo_gemm_f64(qr, sr, fmt, qr, sr, fmt, rows, rows, K, c, t) != 0) return 3;
                int64_t ms[2] = {0, rows - 1}, ns[2] = {rows - 1, 0};
                if (mxo_gemm_f64_at(qr, sr, fmt, qr, sr, fmt, rows, rows, K, ms, ns, 2, c, t) != 0)
                  return 4;
                free(c);
                free(t);
              }
              free(qr);
              free(sr);
              free(qc);
              free(sc);
            }
    free(x);
    free(xb);
  }
  for (unsigned code = 0; code < 256; code++)
    for (int fmt = 0; fmt < 6; fmt++) (void)mxo_elem_value(fmt, code);
  printf("oracle: all entry points ran clean\n");
  return 0;
}
