/*
 * libternary: the 1.58-bit (ternary-weight) linear layer on AMD Instinct MI355X
 * (gfx950).
 *
 * The operation is the one "1.58-bit FLUX" (arXiv 2412.18653) builds its
 * custom kernel around: every weight of a linear layer is restricted to
 * {-1, 0, +1} in the manner of BitNet b1.58 (abstract; section 1
 * Introduction; section 2 Related Work), the ternary weights are stored as
 * 2-bit signed integers instead of 16-bit values (section 1, storage
 * paragraph), and the activations stay unquantized (section 4, limitation on
 * speed).  The library turns full-precision weights into ternary codes and a
 * per-output-channel scale, packs them four to a byte, and computes
 * Y = (X . T^T) (.) s with bf16 X and Y.
 *
 * Conventions shared by every call:
 *  - All data pointers are DEVICE pointers owned by the caller.  The library
 *    allocates and frees no device memory.  It keeps none either, with one
 *    exception: the fixed array of tern_gemm_dx_static (below), which each
 *    GPU that runs the library holds until the process ends.
 *  - Matrices are row-major.  Leading dimensions (ld*) count elements, except
 *    ldp, which counts bytes.
 *  - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL is the default stream) and returns after enqueueing.  Faults inside
 *    a kernel surface at the caller's next synchronisation with that stream.
 *  - Arguments are validated on the host, before anything is enqueued, in
 *    this order: dtype or activation kind, sizes, (no-op check), null
 *    pointers, leading dimensions, alignment.  A call whose output is empty (a zero size) is a
 *    no-op that returns TERN_OK without touching any pointer.
 *  - A kernel launch that the HIP runtime rejects returns TERN_ERR_HIP.
 *  - Outputs must not overlap inputs.  Calls are re-entrant and thread-safe,
 *    and calls on different streams may run at the same time on one GPU: no
 *    state is shared between calls (tern_gemm_dx_static's array aside).
 *  - Inputs are assumed finite; results for NaN or infinite inputs are
 *    unspecified.
 */
#ifndef TERNARY_H_
#define TERNARY_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TERN_OK = 0,
  TERN_ERR_NULL = 1,   /* a required pointer is NULL */
  TERN_ERR_SHAPE = 2,  /* a size is negative or outside the supported range */
  TERN_ERR_ALIGN = 3,  /* a pointer or leading dimension breaks an alignment rule */
  TERN_ERR_STRIDE = 4, /* a leading dimension is too short for its row, or too long */
  TERN_ERR_DTYPE = 5,  /* unknown element type */
  TERN_ERR_HIP = 6,    /* the HIP runtime rejected a launch */
  TERN_ERR_ARG = 7     /* an argument is outside its set of allowed values */
} tern_status;

typedef enum { TERN_F32 = 0, TERN_BF16 = 1 } tern_dtype;

/* Largest row length tern_quantize accepts (see the scale definition below). */
#define TERN_QUANTIZE_MAX_K 32768

/*
 * tern_quantize: absmean ternarization, one scale per output channel.
 *
 * Definition ("1.58-bit FLUX", section 1: weights restricted to {+1, 0, -1}
 * as in BitNet b1.58; the pages give no formula, and the per-output-channel
 * absmean rule below is the reading used):
 *   s_n  = mean_k |w[n][k]|
 *   T_nk = clip(round(w[n][k] / s_n), -1, 1), ties to even, so |w|/s_n = 1/2
 *          gives 0; decided by the exact test 2|w| > s_n (no division).
 *   A row of zeros gives s_n = 0 and T = 0.
 * To make s_n independent of summation order (bit-identical on any device),
 * the mean is taken in 64-bit fixed point: with E = floor(log2(max_k |w|)),
 *   s_n = fp32( fp64(sum_k floor(|w| * 2^(48-E))) * 2^(E-48) / K ),
 * every rounding being IEEE round-to-nearest-even.  This equals the correctly
 * rounded mean except when the exact mean lies within 2^-33 (relative) of a
 * point half-way between two fp32 values.
 *
 *   w      [n, ldw] fp32 (w_dtype = TERN_F32) or bf16 (TERN_BF16), read only
 *   t      [n, ldt] int8 output, values in {-1, 0, +1}; columns >= k untouched
 *   s      [n] fp32 output
 * Sizes: 0 <= n <= 2^31 - 1, 1 <= k <= TERN_QUANTIZE_MAX_K (else
 * TERN_ERR_SHAPE); n == 0 is a no-op.  ldw >= k and ldt >= k (else
 * TERN_ERR_STRIDE).  w aligned to its element size and s to 4 bytes (else
 * TERN_ERR_ALIGN).
 */
tern_status tern_quantize(const void* w, tern_dtype w_dtype, int64_t n, int64_t k, int64_t ldw,
                          int8_t* t, int64_t ldt, float* s, void* stream);

/*
 * tern_pack: 2-bit storage of ternary weights, four per byte
 * ("1.58-bit FLUX", section 1: the 1.58-bit weights are stored as 2-bit
 * signed integers).  Reading of the layout: weight k of a row sits in bits
 * 2*(k%4) and 2*(k%4)+1 of byte k/4 of that row, as the low two bits of its
 * two's-complement value (+1 -> 01, 0 -> 00, -1 -> 11).
 *
 *   t  [n, ldt] int8 input; only the low two bits of each value are used
 *      (values outside {-1, 0, +1} are not rejected)
 *   p  [n, ldp] uint8 output; bytes 0 .. ceil(k/4)-1 of each row are written,
 *      fields past column k-1 in the last byte are 00, and bytes from
 *      ceil(k/4) to ldp-1 are left untouched
 * Sizes: n, k >= 0; a zero size is a no-op.  ldt >= k, ldp >= ceil(k/4).
 */
tern_status tern_pack(const int8_t* t, int64_t n, int64_t k, int64_t ldt, uint8_t* p, int64_t ldp,
                      void* stream);

/*
 * tern_quantize_pack: tern_quantize and tern_pack of its result in one pass
 * over the weights, for the conversion of a full-precision layer into the
 * stored 2-bit form ("1.58-bit FLUX", section 1: ternary weights as in
 * BitNet b1.58, stored as 2-bit signed integers).  The outputs are
 * bit-identical to tern_quantize followed by tern_pack; the codes are not
 * read back from memory, so the int8 matrix may be skipped.
 *
 *   w, w_dtype, n, k, ldw, s: as tern_quantize
 *   t  [n, ldt] int8 output as tern_quantize, or NULL to skip it (ldt is then
 *      ignored)
 *   p  [n, ldp] uint8 output as tern_pack: bytes 0 .. ceil(k/4)-1 of each row
 *      written, fields past column k-1 zero, bytes from ceil(k/4) on untouched
 * Sizes as tern_quantize (TERN_ERR_SHAPE).  ldw >= k, ldt >= k when t is not
 * NULL, ldp >= ceil(k/4) (else TERN_ERR_STRIDE).  w, p and s must not be NULL
 * (TERN_ERR_NULL).  Alignment as tern_quantize (TERN_ERR_ALIGN).
 */
tern_status tern_quantize_pack(const void* w, tern_dtype w_dtype, int64_t n, int64_t k,
                               int64_t ldw, int8_t* t, int64_t ldt, uint8_t* p, int64_t ldp,
                               float* s, void* stream);

/*
 * tern_unpack: the inverse of tern_pack.  Each 2-bit field is sign-extended:
 * 00 -> 0, 01 -> +1, 11 -> -1, and the unused code 10 -> -2 (so that a
 * corrupted code stays visible).
 *
 *   p  [n, ldp] uint8 input; t [n, ldt] int8 output, columns >= k untouched
 * Sizes: n, k >= 0; a zero size is a no-op.  ldp >= ceil(k/4), ldt >= k.
 */
tern_status tern_unpack(const uint8_t* p, int64_t n, int64_t k, int64_t ldp, int8_t* t,
                        int64_t ldt, void* stream);

/*
 * tern_gemm: the ternary linear layer with a fused scale epilogue
 * ("1.58-bit FLUX", section 1 contributions and section 3.2 Results: the
 * efficient linear kernel for 1.58-bit weights; section 4: activations are
 * not quantized).
 *
 *   Y[m][n] = bf16( fp32(acc[m][n]) * s[n] ),  acc[m][n] = sum_k X[m][k] * T[n][k]
 *
 * with T decoded from p as tern_unpack does, the products exact, acc an fp32
 * sum in an unspecified order, and one round-to-nearest-even conversion to
 * bf16.  Codes 10 give an unspecified result.  No bias is added.
 *
 *   x  [m, ldx] bf16 activations
 *   p  [n, ldp] packed weights, as written by tern_pack for a row length k
 *   s  [n] fp32 per-output-channel scales
 *   y  [m, ldy] bf16 output; columns >= n untouched
 * Sizes: m, n, k >= 0 and k % 64 == 0 (else TERN_ERR_SHAPE); m == 0 or
 * n == 0 is a no-op; k == 0 writes zeros.  m, n <= 2^31 - 1,
 * k <= 2^31 - 64 and ceil(m/64) * ceil(n/128) <= 2^31 - 1.
 * ldx >= k, ldp >= k/4, ldy >= n, and ldx < 2^23, ldp < 2^24, ldy < 2^31
 * (else TERN_ERR_STRIDE).
 * Alignment (else TERN_ERR_ALIGN): x and p 16-byte aligned, ldx % 8 == 0,
 * ldp % 16 == 0; y 2-byte aligned; s 4-byte aligned.
 */
tern_status tern_gemm(const void* x_bf16, int64_t m, int64_t k, int64_t ldx, const uint8_t* p,
                      int64_t n, int64_t ldp, const float* s, void* y_bf16, int64_t ldy,
                      void* stream);

/* Activation of the fused epilogue of tern_gemm_ex. */
typedef enum { TERN_ACT_NONE = 0, TERN_ACT_GELU_TANH = 1 } tern_act;

/*
 * tern_gemm_ex: tern_gemm with a fused bias and activation, for the layers
 * that the ternary linear feeds in a diffusion transformer: the MLP
 * up-projection followed by GELU, and the single-stream in-projection whose
 * trailing (MLP) columns are followed by GELU.  The pages give the layer
 * without either ("1.58-bit FLUX", section 1 and section 4); the activation is
 * the tanh form of GELU (Hendrycks and Gimpel),
 *   gelu(z) = z/2 * (1 + tanh(sqrt(2/pi) * (z + 0.044715 z^3))).
 *
 *   Y[m][n] = bf16( f_n( fp32(acc[m][n] * s[n]) + b[n] ) )
 *
 * with acc as in tern_gemm, b[n] = bias[n] (0 when bias is NULL), the sum in
 * fp32, and f_n = gelu evaluated in fp32 (accurate to a few units in the
 * last place) when act = TERN_ACT_GELU_TANH and n >= act_from, else the
 * identity.  tern_gemm_ex(..., NULL, TERN_ACT_NONE, 0, ...) is tern_gemm.
 *
 *   bias      NULL or [n] fp32, 4-byte aligned (else TERN_ERR_ALIGN)
 *   act       TERN_ACT_NONE or TERN_ACT_GELU_TANH (else TERN_ERR_ARG)
 *   act_from  with TERN_ACT_GELU_TANH: 0 <= act_from <= n (else TERN_ERR_ARG);
 *             ignored with TERN_ACT_NONE
 * All other arguments, sizes and rules as tern_gemm; k == 0 writes
 * bf16(f_n(b[n])).
 */
tern_status tern_gemm_ex(const void* x_bf16, int64_t m, int64_t k, int64_t ldx, const uint8_t* p,
                         int64_t n, int64_t ldp, const float* s, const float* bias, tern_act act,
                         int64_t act_from, void* y_bf16, int64_t ldy, void* stream);

/* Static, never-NULL description of a status code. */
const char* tern_status_string(tern_status status);

/*
 * Training in the loop ("TerDiT: Ternary Diffusion Models with Transformers",
 * abstract: quantization-aware training of ternary DiT weights; the pages
 * give no formula).  For the layer Y = (X . T^T) (.) s the gradient with
 * respect to its input is dX = (dY (.) s) . T, a ternary GEMM that contracts
 * over the output channels n.  The codes are used packed along n for it.
 */

/*
 * tern_pack_transposed: the codes of packed weights re-packed along n.
 *
 *   p   [n, ldp] uint8 input, packed as tern_pack writes it for a row length
 *       k (row n holds T[n][0..k-1])
 *   pt  [k, ldpt] uint8 output: row k holds T[0..n-1][k], four codes per
 *       byte, code n in bits 2(n%4) .. 2(n%4)+1 of byte n/4 (the tern_pack
 *       layout with the roles of n and k exchanged); fields past n in the
 *       last byte are 00, bytes from ceil(n/4) to ldpt-1 are left untouched
 * Sizes: 0 <= n, k <= 2^31 - 1 (else TERN_ERR_SHAPE); a zero size is a no-op.
 * ldp >= ceil(k/4), ldpt >= ceil(n/4) (else TERN_ERR_STRIDE).  p and pt must
 * not be NULL (TERN_ERR_NULL).
 */
tern_status tern_pack_transposed(const uint8_t* p, int64_t n, int64_t k, int64_t ldp, uint8_t* pt,
                                 int64_t ldpt, void* stream);

/*
 * tern_gemm_dx: the input gradient of the ternary layer.
 *
 *   u[m][j]  = bf16( fp32(dy[m][j]) * s[j] )          (round to nearest even)
 *   dx[m][c] = bf16( sum_j u[m][j] * T[j][c] )
 *
 * the sum over the n output channels j of the forward layer in fp32 in an
 * unspecified order, with one round-to-nearest-even conversion at the end.
 *
 *   dy  [m, lddy] bf16 gradient of the layer's output Y (m tokens, n channels)
 *   pt  [k, ldpt] the layer's codes packed along n, as tern_pack_transposed
 *       writes them (k = the layer's input width)
 *   s   [n] fp32 the layer's per-channel scales
 *   u   [m, ldu] bf16 workspace, owned by the caller and overwritten with the
 *       scaled gradient (it may be read afterwards)
 *   dx  [m, lddx] bf16 output; columns >= k untouched
 * Sizes: m, n, k >= 0 and n % 64 == 0 (else TERN_ERR_SHAPE); m == 0 or
 * k == 0 is a no-op; n == 0 writes zeros.  m, k <= 2^31 - 1,
 * n <= 2^31 - 64, ceil(m/64) * ceil(k/128) <= 2^31 - 1.
 * lddy >= n, ldu >= n, ldpt >= n/4, lddx >= k, and ldu < 2^23, ldpt < 2^24,
 * lddx < 2^31 (else TERN_ERR_STRIDE).  pt and dx must not be NULL, nor dy, s
 * and u unless n == 0 (TERN_ERR_NULL).  Alignment (else TERN_ERR_ALIGN): u
 * and pt 16-byte aligned, ldu % 8 == 0, ldpt % 16 == 0; dy and dx 2-byte
 * aligned; s 4-byte aligned; with n == 0 the rules on dy, s, u and ldu (not
 * read then) do not apply.  u must not overlap dy, pt, s or dx.  Two
 * launches on `stream`: the scaling, then the product (the kernels of
 * tern_gemm with unit scales).
 */
tern_status tern_gemm_dx(const void* dy_bf16, int64_t m, int64_t n, int64_t lddy,
                         const uint8_t* pt, int64_t k, int64_t ldpt, const float* s,
                         void* u_bf16, int64_t ldu, void* dx_bf16, int64_t lddx, void* stream);

/*
 * tern_gemm_dw: the gradient of the layer's latent full-precision weights, for
 * training the ternary weights in the loop ("TerDiT: Ternary Diffusion Models
 * with Transformers", abstract: quantization-aware training of ternary DiTs;
 * the pages give no formula).  The forward layer is Y = X . (s (.) T)^T, the
 * quantized weight s_n T_nk standing in for the latent weight w_nk; the
 * straight-through estimator passes the gradient of the quantized weight to
 * the latent one unchanged, so
 *
 *   dw[j][c] = (accumulate ? dw[j][c] : 0) + sum_i dy[i][j] * x[i][c]
 *
 * with the products exact and the sum in fp32, in an order that is fixed for
 * given sizes (repeated calls give identical bits).  The ternary codes and the
 * scales do not enter.
 *
 *   dy  [m, lddy] bf16 gradient of the layer output Y (m tokens, n channels)
 *   x   [m, ldx] bf16 layer input X (k input features)
 *   dw  [n, lddw] fp32 output (the latent weights' gradient, row n = output
 *       channel); with accumulate != 0 it is added into (gradient
 *       accumulation over micro-batches); columns >= k untouched
 * Sizes: 0 <= m, n, k <= 2^31 - 1 and ceil(n/128) * ceil(k/128) <= 2^31 - 1,
 * (m - 1) * lddy + n and (m - 1) * ldx + k, each with the width rounded up to
 * a multiple of 8, below 2^31 (else TERN_ERR_SHAPE);
 * n == 0 or k == 0 is a no-op; m == 0 writes zeros (nothing with accumulate).
 * lddw >= k (and lddw < 2^31), and with m > 0: lddy >= n, ldx >= k (else
 * TERN_ERR_STRIDE).  dw must not be NULL, nor dy and x when m > 0
 * (TERN_ERR_NULL).  Alignment (else TERN_ERR_ALIGN): dw 4-byte aligned; with
 * m > 0, dy and x 16-byte aligned and lddy % 8 == 0, ldx % 8 == 0.  Rows of
 * dy and x are read in whole 16-byte pieces: the last row must be readable up
 * to its width rounded up to a multiple of 8 elements (true of every pitched
 * matrix, whose rows span lddy or ldx elements).  dw must not overlap dy or x.
 */
tern_status tern_gemm_dw(const void* dy_bf16, int64_t m, int64_t n, int64_t lddy,
                         const void* x_bf16, int64_t k, int64_t ldx, float* dw, int64_t lddw,
                         int accumulate, void* stream);

/* Largest m * n that tern_gemm_dx_static accepts: its array holds this many
 * bf16 values (128 MiB) on each GPU. */
#define TERN_GEMM_DX_STATIC_MAX_ELEMS 67108864

/*
 * tern_gemm_dx_static: tern_gemm_dx without a caller workspace, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving or training loops, and harnesses that forbid hipMalloc.  The
 * scaled gradient u is written to a fixed device array of the library
 * instead (row pitch n); the call itself allocates nothing.
 *
 *   u[m][j]  = bf16( fp32(dy[m][j]) * s[j] ),   dx[m][c] = bf16( sum_j u[m][j] * T[j][c] )
 *
 * exactly as tern_gemm_dx (same kernels, bit-identical dx).
 *
 *   dy, pt, s, dx and their sizes and leading dimensions: as tern_gemm_dx
 * Sizes as tern_gemm_dx, and m * n <= TERN_GEMM_DX_STATIC_MAX_ELEMS (else
 * TERN_ERR_SHAPE).  Strides, nulls and alignment as tern_gemm_dx without the
 * rules on u and ldu (n < 2^23 takes the place of ldu < 2^23).
 *
 * The array: 128 MiB per GPU, allocated when the library's device code is
 * loaded on that GPU and held until the process ends.  Its device address on
 * the GPU of `stream` is looked up on the first call there (a failure of that
 * lookup returns TERN_ERR_HIP).  Every call on one GPU uses that GPU's one
 * array and leaves its contents (the last call's u) behind: calls that
 * overlap in time on one GPU (on different streams, or from different host
 * threads without ordering) race on it and give undefined results.  Calls on
 * one stream, or otherwise ordered, are safe.
 */
tern_status tern_gemm_dx_static(const void* dy_bf16, int64_t m, int64_t n, int64_t lddy,
                                const uint8_t* pt, int64_t k, int64_t ldpt, const float* s,
                                void* dx_bf16, int64_t lddx, void* stream);

/*
 * 8-bit activations (W1.58-A8).  "1.58-bit FLUX" (section 4, limitation on
 * speed) names the unquantized activations as the reason its latency barely
 * improved, and gives no activation quantizer.  These calls use absmax
 * quantization per token (the BitNet b1.58 family the paper follows,
 * section 1), with the ternary weights unchanged, on the int8 matrix cores.
 */

/*
 * tern_quantize_act: per-token int8 activations.
 *
 *   g_m      = max( max_k |x[m][k]|, 1e-5f )
 *   q[m][k]  = rint( fp32( x[m][k] * fp32(127 / g_m) ) )   (ties to even)
 *   xs[m]    = fp32( g_m / 127 )
 *
 * with both quotients correctly rounded to fp32; |q| <= 127.  The floor
 * (the fp32 value nearest 1e-5) keeps 127 / g finite; a row of zeros gives
 * q = 0 and xs = fp32(1e-5f / 127), and so does k == 0 for xs.
 *
 *   x   [m, ldx] bf16 activations
 *   q   [m, ldq] int8 output codes; columns >= k untouched
 *   xs  [m] fp32 output per-token scales
 * Sizes: 0 <= m, k <= 2^31 - 1 (else TERN_ERR_SHAPE); m == 0 is a no-op;
 * k == 0 writes xs only (x and q are not read and may be NULL).  ldx >= k,
 * ldq >= k (else TERN_ERR_STRIDE).  Alignment (else TERN_ERR_ALIGN): x 2-byte
 * aligned, xs 4-byte aligned.
 */
tern_status tern_quantize_act(const void* x_bf16, int64_t m, int64_t k, int64_t ldx, int8_t* q,
                              int64_t ldq, float* xs, void* stream);

/*
 * tern_pack_a8: packed codes re-arranged for tern_gemm_a8.  Within every
 * 32-bit little-endian word of a row (codes 16 w .. 16 w + 15), field 4 i + j
 * (bits 2(4i+j) .. 2(4i+j)+1) of the output holds code 4 j + i of the word:
 * the 2-bit fields transposed as a 4 x 4 matrix.  The arrangement is its
 * own inverse.
 *
 *   p   [n, ldp] uint8, packed as tern_pack writes it for a row length k
 *   p8  [n, ldp8] uint8 output; bytes k/4 .. ldp8 - 1 of a row untouched.
 *       p8 == p with ldp8 == ldp converts in place; otherwise the two must
 *       not overlap.
 * Sizes: 0 <= n, k <= 2^31 - 1 and k % 16 == 0 (else TERN_ERR_SHAPE); a zero
 * size is a no-op.  ldp, ldp8 >= k/4 (else TERN_ERR_STRIDE).  Alignment
 * (else TERN_ERR_ALIGN): p and p8 4-byte aligned, ldp % 4 == 0,
 * ldp8 % 4 == 0.
 */
tern_status tern_pack_a8(const uint8_t* p, int64_t n, int64_t k, int64_t ldp, uint8_t* p8,
                         int64_t ldp8, void* stream);

/*
 * tern_gemm_a8: the ternary layer on int8 activations.
 *
 *   Y[m][n] = bf16( f_n( fp32( fp32(acc[m][n]) * fp32(s[n] / 64) ) * xs[m] + b[n] ) ),
 *   acc[m][n] = 64 * sum_k q[m][k] * T[n][k]       (exact int32)
 *
 * with T decoded from p8, one round-to-nearest-even conversion to bf16, b and
 * f_n as in tern_gemm_ex (bias NULL and TERN_ACT_NONE: the plain layer).  The
 * fp32 steps are exact but for at most three roundings of 2^-24 relative
 * (acc converted, the two products) before the bf16 rounding.
 *
 *   q    [m, ldq] int8 activations, as tern_quantize_act writes them
 *   xs   [m] fp32 per-token scales, as tern_quantize_act writes them
 *   p8   [n, ldp8] codes arranged by tern_pack_a8 for a row length k
 *   s    [n] fp32 per-output-channel scales
 *   bias, act, act_from   as tern_gemm_ex
 *   y    [m, ldy] bf16 output; columns >= n untouched
 * Sizes: m, n, k >= 0 and k % 128 == 0 (else TERN_ERR_SHAPE); m == 0 or
 * n == 0 is a no-op; k == 0 writes bf16(f_n(b[n])).  m, n <= 2^31 - 1,
 * k <= 2^18 (the int32 sums cannot overflow) and
 * ceil(m/64) * ceil(n/128) <= 2^31 - 1.
 * ldq >= k, ldp8 >= k/4, ldy >= n, and ldq < 2^24, ldp8 < 2^24, ldy < 2^31
 * (else TERN_ERR_STRIDE).  Alignment (else TERN_ERR_ALIGN): q and p8 16-byte
 * aligned, ldq % 16 == 0, ldp8 % 16 == 0; y 2-byte aligned; xs, s and bias
 * 4-byte aligned.
 */
tern_status tern_gemm_a8(const int8_t* q, int64_t m, int64_t k, int64_t ldq, const float* xs,
                         const uint8_t* p8, int64_t n, int64_t ldp8, const float* s,
                         const float* bias, tern_act act, int64_t act_from, void* y_bf16,
                         int64_t ldy, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TERNARY_H_ */
