/*
 * CPU oracle for the 1.58-bit linear layer: test infrastructure only.
 *
 * This file is the plain, slow reference that the GPU library is checked
 * against.  Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark load it; the GPU library never does, and the two share no
 * code, header, table or helper.  Everything here is scalar C with double
 * accumulation, no SIMD intrinsics, no BLAS and no fast-math.
 *
 * What it computes, and where the definition comes from:
 *
 *  - Ternary weights in {-1, 0, +1}, BitNet-b1.58 style ("1.58-bit FLUX",
 *    abstract and section 1 Introduction; section 2 Related Work names
 *    BitNet b1.58).  The pages give no formula; the reading used is the
 *    per-output-channel absmean rule s_n = mean_k |w_nk|,
 *    T = clip(round(w / s_n), -1, 1) with round-half-to-even.
 *  - Storage as 2-bit signed integers, four per byte ("1.58-bit FLUX",
 *    section 1 Introduction, the storage paragraph).
 *  - The layer output Y = (X . T^T) (.) s for unquantized bf16 activations
 *    ("1.58-bit FLUX", section 4, limitation on speed: activations are not
 *    quantized).
 *  - An epilogue variant of that output: a per-channel bias and the
 *    tanh-form GELU on a trailing range of columns (oracle_epilogue; not on
 *    the pages: the activation of the FLUX MLP, the reading is stated there).
 *  - An 8-bit-activation variant of the layer (W1.58-A8; "1.58-bit FLUX",
 *    section 4 names unquantized activations as the reason its latency did
 *    not improve; the pages give no activation quantizer): each token's
 *    activations are scaled by 127 / max|x| and rounded to int8
 *    (oracle_quantize_act), and the layer is s_n * (max|x_m| / 127) times the
 *    exact integer sum of q . T (oracle_gemm_a8); max|x| is floored at 1e-5.  oracle_pack_a8 writes the
 *    codes with the four 2-bit fields of each 4-code group of every 16-code
 *    word exchanged across groups (a 4 x 4 transposition of the fields).
 *  - The gradient of the layer with respect to its input, for training the
 *    ternary weights in the loop ("TerDiT", abstract: quantization-aware
 *    training of ternary DiTs; the pages give no formula): with
 *    Y = (X . T^T) (.) s, dX = (dY (.) s) . T.  oracle_scale_grad forms the
 *    scaled gradient u = bf16(dY (.) s) as a bf16 operand, oracle_gemm_dx the
 *    unrounded sum over n of u . T (T in the forward's packed layout).
 *  - The gradient of the latent full-precision weights for that training,
 *    under the straight-through reading (the quantizer passes the gradient
 *    of the quantized weight s_n T_nk to the latent weight unchanged):
 *    oracle_gemm_dw, dW = dY^T . X, unrounded.
 *
 * Readings where the pages are silent (all listed in the design notes):
 *  - the mean is taken in 64-bit fixed point relative to the row's largest
 *    binade, so that its value does not depend on summation order
 *    (oracle_quantize, steps 3-5);
 *  - the half-way case |w|/s = 1/2 rounds to 0 (ties to even), decided by the
 *    exact test 2|w| > s instead of a division;
 *  - a row of zeros gets s = 0 and T = 0 (no epsilon);
 *  - 2-bit codes are two's complement (+1 = 01, 0 = 00, -1 = 11), packed
 *    along K, least significant bits first; code 10 decodes to -2.
 *
 * Parity pins for every function live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* bf16 -> fp32: a bf16 value is the upper half of an fp32 bit pattern. */
static float bf16_bits_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static float load_weight(const void* w, int w_is_bf16, int64_t idx) {
  if (w_is_bf16) return bf16_bits_to_float(((const uint16_t*)w)[idx]);
  return ((const float*)w)[idx];
}

/*
 * Absmean ternarization of one row (per output channel).
 *
 * Steps, for row n with K entries:
 *  1. a_k = |w_k| in fp32 (bf16 input widened exactly first).
 *  2. A = max_k a_k.  If A == 0 the row is all zeros: s = 0, T = 0.
 *  3. E = floor(log2 A), exactly, from frexp: A = f * 2^e with f in [1/2, 1).
 *  4. q_k = floor(a_k * 2^(48 - E)) as an unsigned 64-bit integer.  The
 *     scaling by a power of two is exact in double and floor is the only
 *     rounding; q_k < 2^49, so the sum below cannot overflow for K <= 32768.
 *  5. s = (float)( (double)Q * 2^(E - 48) / (double)K ), Q = sum_k q_k.
 *  6. T_k = +1 or -1 (sign of w_k) when 2 * a_k > s, else 0.  This is
 *     clip(round(w/s), -1, 1) with ties to even: |w|/s > 1/2 gives +-1, and
 *     |w|/s == 1/2 rounds to 0.
 */
static void quantize_row(const void* w, int w_is_bf16, int64_t row_off, int64_t k,
                         int8_t* t_row, float* s_out) {
  float amax = 0.0f;
  for (int64_t i = 0; i < k; ++i) {
    float a = fabsf(load_weight(w, w_is_bf16, row_off + i));
    if (a > amax) amax = a;
  }
  if (amax == 0.0f) {
    *s_out = 0.0f;
    for (int64_t i = 0; i < k; ++i) t_row[i] = 0;
    return;
  }
  int e;
  (void)frexp((double)amax, &e);
  int E = e - 1;

  uint64_t Q = 0;
  for (int64_t i = 0; i < k; ++i) {
    double a = (double)fabsf(load_weight(w, w_is_bf16, row_off + i));
    Q += (uint64_t)floor(ldexp(a, 48 - E));
  }
  double mean = ldexp((double)Q, E - 48) / (double)k;
  float s = (float)mean;
  *s_out = s;

  for (int64_t i = 0; i < k; ++i) {
    float wv = load_weight(w, w_is_bf16, row_off + i);
    float a = fabsf(wv);
    if (2.0f * a > s)
      t_row[i] = (wv < 0.0f) ? (int8_t)-1 : (int8_t)1;
    else
      t_row[i] = 0;
  }
}

/* w_dtype: 0 = fp32, 1 = bf16 (raw 16-bit patterns). */
int oracle_quantize(const void* w, int w_dtype, int64_t n, int64_t k, int64_t ldw,
                    int8_t* t, int64_t ldt, float* s) {
  if (n < 0 || k < 1 || k > 32768 || ldw < k || ldt < k) return ORACLE_BAD_ARG;
  if (w_dtype != 0 && w_dtype != 1) return ORACLE_BAD_ARG;
  for (int64_t r = 0; r < n; ++r)
    quantize_row(w, w_dtype == 1, r * ldw, k, t + r * ldt, s + r);
  return ORACLE_OK;
}

/*
 * 2-bit packing, four weights per byte along K, least significant first:
 * weight k sits in bits 2*(k%4) .. 2*(k%4)+1 of byte k/4 of its row, as the
 * low two bits of its two's-complement value (+1 -> 01, 0 -> 00, -1 -> 11).
 * Positions past the end of a row (K % 4 != 0) hold code 00.
 */
int oracle_pack(const int8_t* t, int64_t n, int64_t k, int64_t ldt, uint8_t* p, int64_t ldp) {
  int64_t nbytes = (k + 3) / 4;
  if (n < 0 || k < 0 || ldt < k || ldp < nbytes) return ORACLE_BAD_ARG;
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t j = 0; j < nbytes; ++j) {
      unsigned byte = 0;
      for (int i = 0; i < 4; ++i) {
        int64_t kk = 4 * j + i;
        unsigned code = 0;
        if (kk < k) code = (unsigned)(uint8_t)t[r * ldt + kk] & 3u;
        byte |= code << (2 * i);
      }
      p[r * ldp + j] = (uint8_t)byte;
    }
  }
  return ORACLE_OK;
}

/* Sign-extend a 2-bit field: 00 -> 0, 01 -> +1, 10 -> -2, 11 -> -1. */
static int decode_code(unsigned code) {
  return (code & 2u) ? (int)code - 4 : (int)code;
}

int oracle_unpack(const uint8_t* p, int64_t n, int64_t k, int64_t ldp, int8_t* t, int64_t ldt) {
  if (n < 0 || k < 0 || ldp < (k + 3) / 4 || ldt < k) return ORACLE_BAD_ARG;
  for (int64_t r = 0; r < n; ++r)
    for (int64_t kk = 0; kk < k; ++kk) {
      unsigned code = (p[r * ldp + kk / 4] >> (2 * (kk % 4))) & 3u;
      t[r * ldt + kk] = (int8_t)decode_code(code);
    }
  return ORACLE_OK;
}

/*
 * Layer output, unrounded: y[m][n] = s_n * sum_k x[m][k] * T[n][k], with x the
 * bf16 activations widened exactly, T decoded from the packed bytes, the sum
 * taken in double in ascending k, and one double multiply by s_n.  The result
 * is left in double: the GPU's bf16 output is compared against it with a
 * tolerance, never against a rounded copy.
 *
 * Work is split over output columns n across threads; each thread decodes one
 * weight row at a time and runs it against every activation row.
 */
typedef struct {
  const double* xd;  /* m x k, widened activations */
  int64_t m, k;
  const uint8_t* p;
  int64_t ldp;
  const float* s;
  double* y;
  int64_t ldy;
  int64_t n_begin, n_end;
} gemm_job;

static void* gemm_worker(void* arg) {
  gemm_job* j = (gemm_job*)arg;
  int8_t* trow = (int8_t*)malloc((size_t)(j->k > 0 ? j->k : 1));
  if (!trow) return (void*)1;
  for (int64_t n = j->n_begin; n < j->n_end; ++n) {
    for (int64_t kk = 0; kk < j->k; ++kk) {
      unsigned code = (j->p[n * j->ldp + kk / 4] >> (2 * (kk % 4))) & 3u;
      trow[kk] = (int8_t)decode_code(code);
    }
    double sn = (double)j->s[n];
    for (int64_t mm = 0; mm < j->m; ++mm) {
      const double* xr = j->xd + mm * j->k;
      double acc = 0.0;
      for (int64_t kk = 0; kk < j->k; ++kk) acc += xr[kk] * (double)trow[kk];
      j->y[mm * j->ldy + n] = sn * acc;
    }
  }
  free(trow);
  return NULL;
}

int oracle_gemm(const uint16_t* x_bf16, int64_t m, int64_t k, int64_t ldx, const uint8_t* p,
                int64_t n, int64_t ldp, const float* s, double* y, int64_t ldy, int nthreads) {
  if (m < 0 || n < 0 || k < 0 || ldx < k || ldp < (k + 3) / 4 || ldy < n) return ORACLE_BAD_ARG;
  if (m == 0 || n == 0) return ORACLE_OK;
  double* xd = (double*)malloc((size_t)(m * (k > 0 ? k : 1)) * sizeof(double));
  if (!xd) return ORACLE_BAD_ARG;
  for (int64_t mm = 0; mm < m; ++mm)
    for (int64_t kk = 0; kk < k; ++kk)
      xd[mm * k + kk] = (double)bf16_bits_to_float(x_bf16[mm * ldx + kk]);

  if (nthreads < 1) nthreads = 1;
  if (nthreads > n) nthreads = (int)n;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  gemm_job* jobs = (gemm_job*)malloc(sizeof(gemm_job) * (size_t)nthreads);
  int rc = ORACLE_OK;
  if (!th || !jobs) rc = ORACLE_BAD_ARG;
  int started = 0;
  for (int i = 0; rc == ORACLE_OK && i < nthreads; ++i) {
    gemm_job jb = {xd, m, k, p, ldp, s, y, ldy, n * i / nthreads, n * (i + 1) / nthreads};
    jobs[i] = jb;
    if (pthread_create(&th[i], NULL, gemm_worker, &jobs[i]) != 0) {
      rc = ORACLE_BAD_ARG;
      break;
    }
    ++started;
  }
  for (int i = 0; i < started; ++i) {
    void* ret = NULL;
    pthread_join(th[i], &ret);
    if (ret != NULL) rc = ORACLE_BAD_ARG;
  }
  free(jobs);
  free(th);
  free(xd);
  return rc;
}

/*
 * Epilogue variant of the layer: bias and activation after the scale.
 *
 *   y[m][n] <- f_n( y[m][n] + b[n] ),  f_n = GELU (tanh form) for n >= act_from
 *                                       f_n = identity otherwise
 *
 * applied in place to an unrounded layer output from oracle_gemm, all in
 * double.  The GELU in its tanh form (Hendrycks and Gimpel) is
 *
 *   gelu(z) = z/2 * (1 + tanh( sqrt(2/pi) * (z + 0.044715 z^3) )),
 *
 * the activation that FLUX's MLP applies after its up-projection.  The pages
 * name no bias and no activation for the ternary layer; this variant is the
 * reading used for the fused epilogues of the MLP up-projection and of the
 * single-stream in-projection (activation on its MLP columns only).
 * bias may be NULL (no bias); act is 0 (none) or 1 (GELU, tanh form).
 */
static double gelu_tanh(double z) {
  const double pi = 3.14159265358979323846;
  const double u = sqrt(2.0 / pi) * (z + 0.044715 * z * z * z);
  return 0.5 * z * (1.0 + tanh(u));
}

int oracle_epilogue(double* y, int64_t m, int64_t n, int64_t ldy, const float* bias, int act,
                    int64_t act_from) {
  if (m < 0 || n < 0 || ldy < n || (act != 0 && act != 1) || act_from < 0 || act_from > n)
    return ORACLE_BAD_ARG;
  for (int64_t mm = 0; mm < m; ++mm)
    for (int64_t nn = 0; nn < n; ++nn) {
      double v = y[mm * ldy + nn];
      if (bias) v += (double)bias[nn];
      if (act == 1 && nn >= act_from) v = gelu_tanh(v);
      y[mm * ldy + nn] = v;
    }
  return ORACLE_OK;
}

/*
 * Scaled output gradient, the operand of the input gradient:
 *
 *   u[m][n] = bf16( fp32(dy[m][n]) * s[n] )
 *
 * one IEEE single-precision product (round to nearest even), then one
 * rounding to bf16, to nearest with ties to even.  The bf16 rounding keeps
 * the upper 16 bits of the single-precision pattern after adding 0x7FFF plus
 * the lowest kept bit (finite values; a carry into the exponent is the
 * correct rounding up, to infinity at the top).
 */
static uint16_t float_to_bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, sizeof b);
  const uint32_t lsb = (b >> 16) & 1u;
  return (uint16_t)((b + 0x7FFFu + lsb) >> 16);
}

int oracle_scale_grad(const uint16_t* dy, int64_t m, int64_t n, int64_t lddy, const float* s,
                      uint16_t* u, int64_t ldu) {
  if (m < 0 || n < 0 || lddy < n || ldu < n) return ORACLE_BAD_ARG;
  for (int64_t mm = 0; mm < m; ++mm)
    for (int64_t nn = 0; nn < n; ++nn) {
      const float prod = bf16_bits_to_float(dy[mm * lddy + nn]) * s[nn];
      u[mm * ldu + nn] = float_to_bf16_rne(prod);
    }
  return ORACLE_OK;
}

/*
 * Input gradient, unrounded: dx[m][k] = sum_{n ascending} u[m][n] * T[n][k],
 * u the bf16 scaled gradient widened exactly, T decoded from the forward's
 * packed bytes (row n, packed along k), the sum in double.  Threads split the
 * output columns k; each thread decodes, for its columns, the whole column of
 * T once and runs it against every gradient row.
 */
typedef struct {
  const double* ud;  /* m x n, widened scaled gradient */
  int64_t m, n;
  const uint8_t* p;
  int64_t ldp;
  double* dx;
  int64_t lddx;
  int64_t k_begin, k_end;
} dx_job;

static void* dx_worker(void* arg) {
  dx_job* j = (dx_job*)arg;
  int8_t* tcol = (int8_t*)malloc((size_t)(j->n > 0 ? j->n : 1));
  if (!tcol) return (void*)1;
  for (int64_t kk = j->k_begin; kk < j->k_end; ++kk) {
    for (int64_t nn = 0; nn < j->n; ++nn) {
      unsigned code = (j->p[nn * j->ldp + kk / 4] >> (2 * (kk % 4))) & 3u;
      tcol[nn] = (int8_t)decode_code(code);
    }
    for (int64_t mm = 0; mm < j->m; ++mm) {
      const double* ur = j->ud + mm * j->n;
      double acc = 0.0;
      for (int64_t nn = 0; nn < j->n; ++nn) acc += ur[nn] * (double)tcol[nn];
      j->dx[mm * j->lddx + kk] = acc;
    }
  }
  free(tcol);
  return NULL;
}

int oracle_gemm_dx(const uint16_t* u, int64_t m, int64_t n, int64_t ldu, const uint8_t* p,
                   int64_t k, int64_t ldp, double* dx, int64_t lddx, int nthreads) {
  if (m < 0 || n < 0 || k < 0 || ldu < n || ldp < (k + 3) / 4 || lddx < k) return ORACLE_BAD_ARG;
  if (m == 0 || k == 0) return ORACLE_OK;
  double* ud = (double*)malloc((size_t)(m * (n > 0 ? n : 1)) * sizeof(double));
  if (!ud) return ORACLE_BAD_ARG;
  for (int64_t mm = 0; mm < m; ++mm)
    for (int64_t nn = 0; nn < n; ++nn) ud[mm * n + nn] = (double)bf16_bits_to_float(u[mm * ldu + nn]);

  if (nthreads < 1) nthreads = 1;
  if (nthreads > k) nthreads = (int)k;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  dx_job* jobs = (dx_job*)malloc(sizeof(dx_job) * (size_t)nthreads);
  int rc = ORACLE_OK;
  if (!th || !jobs) rc = ORACLE_BAD_ARG;
  int started = 0;
  for (int i = 0; rc == ORACLE_OK && i < nthreads; ++i) {
    dx_job jb = {ud, m, n, p, ldp, dx, lddx, k * i / nthreads, k * (i + 1) / nthreads};
    jobs[i] = jb;
    if (pthread_create(&th[i], NULL, dx_worker, &jobs[i]) != 0) {
      rc = ORACLE_BAD_ARG;
      break;
    }
    ++started;
  }
  for (int i = 0; i < started; ++i) {
    void* ret = NULL;
    pthread_join(th[i], &ret);
    if (ret != NULL) rc = ORACLE_BAD_ARG;
  }
  free(jobs);
  free(th);
  free(ud);
  return rc;
}

/*
 * Per-token activation quantization to int8 (absmax):
 *
 *   g_m = max(max_k |x[m][k]|, 1e-5f)   (bf16 values, exact in fp32)
 *   q[m][k] = rint( fp32(x[m][k] * fp32(127 / g_m)) )   (ties to even)
 *   xs[m] = fp32(g_m / 127)
 *
 * each division and product one IEEE single-precision operation.  The floor
 * 1e-5 (the fp32 value nearest to it) keeps 127 / g finite: without it the
 * quotient overflows for rows whose largest magnitude is below 127 / FLT_MAX
 * (about 3.7e-37), which bf16 can hold.  A row of zeros gives q = 0.
 * |x| <= g gives |x * (127 / g)| <= 127 (1 + 2^-23)^2 < 127.5, so q lies in
 * [-127, 127].
 */
int oracle_quantize_act(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, int8_t* q,
                        int64_t ldq, float* xs) {
  if (m < 0 || k < 0 || ldx < k || ldq < k) return ORACLE_BAD_ARG;
  for (int64_t mm = 0; mm < m; ++mm) {
    float g = 0.0f;
    for (int64_t kk = 0; kk < k; ++kk) {
      const float a = fabsf(bf16_bits_to_float(x[mm * ldx + kk]));
      if (a > g) g = a;
    }
    if (g < 1e-5f) g = 1e-5f;
    const float inv = 127.0f / g;
    for (int64_t kk = 0; kk < k; ++kk) {
      const float v = bf16_bits_to_float(x[mm * ldx + kk]) * inv;
      q[mm * ldq + kk] = (int8_t)rintf(v);
    }
    xs[mm] = g / 127.0f;
  }
  return ORACLE_OK;
}

/*
 * The 8-bit-activation layer, unrounded:
 *   y[m][n] = s_n * xs_m * sum_k q[m][k] * T[n][k]
 * with the sum exact in 64-bit integers (ascending k) and the two scale
 * products in double.
 */
int oracle_gemm_a8(const int8_t* q, int64_t m, int64_t k, int64_t ldq, const float* xs,
                   const uint8_t* p, int64_t n, int64_t ldp, const float* s, double* y,
                   int64_t ldy) {
  if (m < 0 || n < 0 || k < 0 || ldq < k || ldp < (k + 3) / 4 || ldy < n) return ORACLE_BAD_ARG;
  int8_t* trow = (int8_t*)malloc((size_t)(k > 0 ? k : 1));
  if (!trow) return ORACLE_BAD_ARG;
  for (int64_t nn = 0; nn < n; ++nn) {
    for (int64_t kk = 0; kk < k; ++kk) {
      unsigned code = (p[nn * ldp + kk / 4] >> (2 * (kk % 4))) & 3u;
      trow[kk] = (int8_t)decode_code(code);
    }
    for (int64_t mm = 0; mm < m; ++mm) {
      int64_t acc = 0;
      for (int64_t kk = 0; kk < k; ++kk) acc += (int64_t)q[mm * ldq + kk] * trow[kk];
      y[mm * ldy + nn] = (double)s[nn] * (double)xs[mm] * (double)acc;
    }
  }
  free(trow);
  return ORACLE_OK;
}

/*
 * Field-transposed packing for the 8-bit-activation layer: in every 32-bit
 * word of a packed row (codes 16 w .. 16 w + 15 of the row), field 4 i + j
 * (bits 2(4i+j) .. 2(4i+j)+1) holds code 4 j + i of the word.  Rows are whole
 * words (k % 16 == 0); bytes k/4 .. ldp8 - 1 of an output row are not written.
 */
int oracle_pack_a8(const uint8_t* p, int64_t n, int64_t k, int64_t ldp, uint8_t* p8,
                   int64_t ldp8) {
  const int64_t nb = k / 4;
  if (n < 0 || k < 0 || k % 16 != 0 || ldp < nb || ldp8 < nb) return ORACLE_BAD_ARG;
  for (int64_t nn = 0; nn < n; ++nn) {
    for (int64_t b = 0; b < nb; ++b) p8[nn * ldp8 + b] = 0;
    for (int64_t c = 0; c < k; ++c) {
      const int64_t w = c / 16, f = c % 16;     /* code f of word w */
      const int64_t i = f % 4, j = f / 4;       /* code 4 j + i -> field 4 i + j */
      const unsigned code = (p[nn * ldp + c / 4] >> (2 * (c % 4))) & 3u;
      const int64_t field = 16 * w + 4 * i + j;
      p8[nn * ldp8 + field / 4] |= (uint8_t)(code << (2 * (field % 4)));
    }
  }
  return ORACLE_OK;
}

/*
 * Gradient of the latent full-precision weights, for quantization-aware
 * training of the ternary layer ("TerDiT", abstract: ternary DiT weights
 * trained in the loop; the pages give no formula).  The forward layer is
 * Y = X . (s (.) T)^T, the quantized weight s_n T_nk standing in for the
 * latent weight w_nk.  The reading used is the straight-through estimator
 * that treats the quantizer as the identity in the backward pass, so the
 * latent weight receives the gradient of the quantized one:
 *
 *   dw[n][k] = sum_{m ascending} dy[m][n] * x[m][k]
 *
 * dy (the gradient of Y, [m, n]) and x (the layer input, [m, k]) bf16,
 * widened exactly, the products and the sum in double, unrounded.  Threads
 * split the output rows n; each thread gathers the column dy[., n] once and
 * runs it against every column of x.
 */
typedef struct {
  const double* dyd;  /* n x m: the widened gradient, transposed */
  const double* xd;   /* k x m: the widened input, transposed */
  int64_t m, k;
  double* dw;
  int64_t lddw;
  int64_t n_begin, n_end;
} dw_job;

static void* dw_worker(void* arg) {
  dw_job* j = (dw_job*)arg;
  for (int64_t nn = j->n_begin; nn < j->n_end; ++nn) {
    const double* g = j->dyd + nn * j->m;
    for (int64_t kk = 0; kk < j->k; ++kk) {
      const double* xc = j->xd + kk * j->m;
      double acc = 0.0;
      for (int64_t mm = 0; mm < j->m; ++mm) acc += g[mm] * xc[mm];
      j->dw[nn * j->lddw + kk] = acc;
    }
  }
  return NULL;
}

int oracle_gemm_dw(const uint16_t* dy, int64_t m, int64_t n, int64_t lddy, const uint16_t* x,
                   int64_t k, int64_t ldx, double* dw, int64_t lddw, int nthreads) {
  if (m < 0 || n < 0 || k < 0 || lddy < n || ldx < k || lddw < k) return ORACLE_BAD_ARG;
  if (n == 0 || k == 0) return ORACLE_OK;
  const int64_t mm1 = m > 0 ? m : 1;
  double* dyd = (double*)malloc((size_t)(n * mm1) * sizeof(double));
  double* xd = (double*)malloc((size_t)(k * mm1) * sizeof(double));
  if (!dyd || !xd) {
    free(dyd);
    free(xd);
    return ORACLE_BAD_ARG;
  }
  for (int64_t mm = 0; mm < m; ++mm) {
    for (int64_t nn = 0; nn < n; ++nn)
      dyd[nn * m + mm] = (double)bf16_bits_to_float(dy[mm * lddy + nn]);
    for (int64_t kk = 0; kk < k; ++kk)
      xd[kk * m + mm] = (double)bf16_bits_to_float(x[mm * ldx + kk]);
  }

  if (nthreads < 1) nthreads = 1;
  if (nthreads > n) nthreads = (int)n;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  dw_job* jobs = (dw_job*)malloc(sizeof(dw_job) * (size_t)nthreads);
  int rc = ORACLE_OK;
  if (!th || !jobs) rc = ORACLE_BAD_ARG;
  int started = 0;
  for (int i = 0; rc == ORACLE_OK && i < nthreads; ++i) {
    dw_job jb = {dyd, xd, m, k, dw, lddw, n * i / nthreads, n * (i + 1) / nthreads};
    jobs[i] = jb;
    if (pthread_create(&th[i], NULL, dw_worker, &jobs[i]) != 0) {
      rc = ORACLE_BAD_ARG;
      break;
    }
    ++started;
  }
  for (int i = 0; i < started; ++i) {
    void* ret = NULL;
    pthread_join(th[i], &ret);
    if (ret != NULL) rc = ORACLE_BAD_ARG;
  }
  free(jobs);
  free(th);
  free(xd);
  free(dyd);
  return rc;
}
