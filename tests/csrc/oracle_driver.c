/*
 * Drives every oracle entry point on small and edge-case shapes (k = 1, k not
 * a multiple of 4, one row, padded leading dimensions, empty sizes, invalid
 * arguments).  Built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_oracle_sanitized.py: any out-of-bounds access, use of freed
 * memory, signed overflow or misaligned access in the oracle aborts the run.
 * Test infrastructure only.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_quantize(const void* w, int w_dtype, int64_t n, int64_t k, int64_t ldw, int8_t* t,
                    int64_t ldt, float* s);
int oracle_pack(const int8_t* t, int64_t n, int64_t k, int64_t ldt, uint8_t* p, int64_t ldp);
int oracle_unpack(const uint8_t* p, int64_t n, int64_t k, int64_t ldp, int8_t* t, int64_t ldt);
int oracle_gemm(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const uint8_t* p, int64_t n,
                int64_t ldp, const float* s, double* y, int64_t ldy, int nthreads);
int oracle_epilogue(double* y, int64_t m, int64_t n, int64_t ldy, const float* bias, int act,
                    int64_t act_from);
int oracle_scale_grad(const uint16_t* dy, int64_t m, int64_t n, int64_t lddy, const float* s,
                      uint16_t* u, int64_t ldu);
int oracle_gemm_dx(const uint16_t* u, int64_t m, int64_t n, int64_t ldu, const uint8_t* p,
                   int64_t k, int64_t ldp, double* dx, int64_t lddx, int nthreads);

int oracle_quantize_act(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, int8_t* q,
                        int64_t ldq, float* xs);
int oracle_gemm_a8(const int8_t* q, int64_t m, int64_t k, int64_t ldq, const float* xs,
                   const uint8_t* p, int64_t n, int64_t ldp, const float* s, double* y,
                   int64_t ldy);
int oracle_pack_a8(const uint8_t* p, int64_t n, int64_t k, int64_t ldp, uint8_t* p8,
                   int64_t ldp8);
int oracle_gemm_dw(const uint16_t* dy, int64_t m, int64_t n, int64_t lddy, const uint16_t* x,
                   int64_t k, int64_t ldx, double* dw, int64_t lddw, int nthreads);

static uint32_t rng = 12345u;
static uint32_t next(void) {
  rng = rng * 1664525u + 1013904223u;
  return rng >> 8;
}
static float frand(void) { return (float)next() / (float)(1u << 24) * 2.0f - 1.0f; }

#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                      \
    }                                                                \
  } while (0)

static int run_shape(int64_t m, int64_t n, int64_t k, int64_t pad, int threads) {
  const int64_t ldw = k + pad, ldt = k + pad, ldp = (k + 3) / 4 + pad, ldx = k + pad;
  const int64_t ldy = n + pad, ldd = n + pad, ldpt = (n + 3) / 4 + pad;
  /* exact-size allocations (+1 so that zero sizes still allocate), so that
     any access past the last row or column is caught */
  float* w = malloc(sizeof(float) * (size_t)(n * ldw + 1));
  uint16_t* wb = malloc(sizeof(uint16_t) * (size_t)(n * ldw + 1));
  int8_t* t = malloc((size_t)(n * ldt + 1));
  int8_t* t2 = malloc((size_t)(n * ldt + 1));
  float* s = malloc(sizeof(float) * (size_t)(n + 1));
  uint8_t* p = malloc((size_t)(n * ldp + 1));
  uint16_t* x = malloc(sizeof(uint16_t) * (size_t)(m * ldx + 1));
  double* y = malloc(sizeof(double) * (size_t)(m * ldy + 1));
  float* bias = malloc(sizeof(float) * (size_t)(n + 1));
  uint16_t* dy = malloc(sizeof(uint16_t) * (size_t)(m * ldd + 1));
  uint16_t* u = malloc(sizeof(uint16_t) * (size_t)(m * ldd + 1));
  double* dx = malloc(sizeof(double) * (size_t)(m * (k + pad) + 1));
  int8_t* q = malloc((size_t)(m * ldx + 1));
  float* xs = malloc(sizeof(float) * (size_t)(m + 1));
  const int64_t k16 = k / 16 * 16, ldp8 = k16 / 4 + pad;
  uint8_t* p8 = malloc((size_t)(n * ldp8 + 1));
  double* dw = malloc(sizeof(double) * (size_t)(n * (k + pad) + 1));
  (void)ldpt;
  for (int64_t i = 0; i < n * ldw; ++i) {
    w[i] = frand() * 0.05f;
    uint32_t b;
    memcpy(&b, &w[i], 4);
    wb[i] = (uint16_t)(b >> 16);
  }
  for (int64_t i = 0; i < m * ldx; ++i) x[i] = (uint16_t)(0x3F00u + (next() & 0xFFu));
  for (int64_t i = 0; i < m * ldd; ++i) dy[i] = (uint16_t)(0xBE00u + (next() & 0x1FFu));
  for (int64_t i = 0; i < n; ++i) bias[i] = frand();
  int rc = 0;
  rc |= oracle_quantize(w, 0, n, k, ldw, t, ldt, s);
  rc |= oracle_quantize(wb, 1, n, k, ldw, t, ldt, s);
  rc |= oracle_pack(t, n, k, ldt, p, ldp);
  rc |= oracle_unpack(p, n, k, ldp, t2, ldt);
  for (int64_t r = 0; r < n; ++r) CHECK(memcmp(t + r * ldt, t2 + r * ldt, (size_t)k) == 0);
  rc |= oracle_gemm(x, m, k, ldx, p, n, ldp, s, y, ldy, threads);
  rc |= oracle_epilogue(y, m, n, ldy, bias, 1, n / 2);
  rc |= oracle_epilogue(y, m, n, ldy, NULL, 0, 0);
  rc |= oracle_scale_grad(dy, m, n, ldd, s, u, ldd);
  rc |= oracle_gemm_dx(u, m, n, ldd, p, k, ldp, dx, k + pad, threads);
  rc |= oracle_quantize_act(x, m, k, ldx, q, ldx, xs);
  rc |= oracle_gemm_a8(q, m, k, ldx, xs, p, n, ldp, s, y, ldy);
  rc |= oracle_pack_a8(p, n, k16, ldp, p8, ldp8);
  rc |= oracle_gemm_dw(dy, m, n, ldd, x, k, ldx, dw, k + pad, threads);
  free(q); free(xs); free(p8); free(dw);
  free(w); free(wb); free(t); free(t2); free(s); free(p); free(x); free(y); free(bias);
  free(dy); free(u); free(dx);
  return rc;
}

int main(void) {
  const int64_t shapes[][3] = {{1, 1, 1}, {3, 5, 7}, {2, 4, 4}, {1, 9, 257}, {17, 33, 130},
                               {0, 3, 8}, {4, 1, 65}, {5, 70, 3}};
  for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i)
    for (int64_t pad = 0; pad <= 3; pad += 3)
      for (int threads = 1; threads <= 3; threads += 2)
        CHECK(run_shape(shapes[i][0], shapes[i][1], shapes[i][2], pad, threads) == 0);
  /* invalid arguments are rejected without touching memory */
  CHECK(oracle_quantize(NULL, 0, 2, 4, 3, NULL, 4, NULL) != 0);   /* ldw < k */
  CHECK(oracle_pack(NULL, 2, 9, 9, NULL, 2) != 0);                /* ldp < ceil(k/4) */
  CHECK(oracle_gemm(NULL, 2, 8, 7, NULL, 2, 2, NULL, NULL, 2, 1) != 0);
  CHECK(oracle_epilogue(NULL, 1, 2, 2, NULL, 2, 0) != 0);
  CHECK(oracle_scale_grad(NULL, 1, 4, 3, NULL, NULL, 4) != 0);
  CHECK(oracle_gemm_dx(NULL, 1, 4, 4, NULL, 8, 1, NULL, 8, 1) != 0);
  CHECK(oracle_quantize_act(NULL, 1, 8, 7, NULL, 8, NULL) != 0);
  CHECK(oracle_gemm_a8(NULL, 1, 8, 8, NULL, NULL, 2, 1, NULL, NULL, 2) != 0);
  CHECK(oracle_pack_a8(NULL, 2, 24, 6, NULL, 6) != 0);             /* k % 16 != 0 */
  CHECK(oracle_gemm_dw(NULL, 2, 4, 3, NULL, 8, 8, NULL, 8, 1) != 0); /* lddy < n */
  printf("oracle driver ok\n");
  return 0;
}
