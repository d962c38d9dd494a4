// C-ABI of libternary (declared in include/ternary.h): host-side argument
// validation, then one asynchronous launch on the caller's stream.  No HIP
// call is made before every argument has been checked, and the library keeps
// no state between calls.
#include "ternary.h"

#include "internal.h"

namespace {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline tern_status from_hip(hipError_t e) { return e == hipSuccess ? TERN_OK : TERN_ERR_HIP; }

constexpr int64_t kMaxInt = 2147483647;  // 2^31 - 1
// The GEMM addresses one 256-row block of X (or of the packed weights) with
// 32-bit byte offsets.
constexpr int64_t kGemmMaxLdx = (int64_t(1) << 23) - 1;
constexpr int64_t kGemmMaxLdp = (int64_t(1) << 24) - 1;

}  // namespace

extern "C" {

tern_status tern_quantize(const void* w, tern_dtype w_dtype, int64_t n, int64_t k, int64_t ldw,
                          int8_t* t, int64_t ldt, float* s, void* stream) {
  if (w_dtype != TERN_F32 && w_dtype != TERN_BF16) return TERN_ERR_DTYPE;
  if (n < 0 || n > kMaxInt || k < 0 || k > TERN_QUANTIZE_MAX_K) return TERN_ERR_SHAPE;
  if (n == 0) return TERN_OK;
  if (k == 0) return TERN_ERR_SHAPE;
  if (w == nullptr || t == nullptr || s == nullptr) return TERN_ERR_NULL;
  if (ldw < k || ldt < k) return TERN_ERR_STRIDE;
  const uintptr_t esz = (w_dtype == TERN_F32) ? 4 : 2;
  if (!aligned(w, esz) || !aligned(s, 4)) return TERN_ERR_ALIGN;
  return from_hip(tern::launch_quantize(w, w_dtype == TERN_BF16, n, k, ldw, t, ldt, s, nullptr, 0,
                                        static_cast<hipStream_t>(stream)));
}

tern_status tern_quantize_pack(const void* w, tern_dtype w_dtype, int64_t n, int64_t k,
                               int64_t ldw, int8_t* t, int64_t ldt, uint8_t* p, int64_t ldp,
                               float* s, void* stream) {
  if (w_dtype != TERN_F32 && w_dtype != TERN_BF16) return TERN_ERR_DTYPE;
  if (n < 0 || n > kMaxInt || k < 0 || k > TERN_QUANTIZE_MAX_K) return TERN_ERR_SHAPE;
  if (n == 0) return TERN_OK;
  if (k == 0) return TERN_ERR_SHAPE;
  if (w == nullptr || p == nullptr || s == nullptr) return TERN_ERR_NULL;
  if (ldw < k || (t != nullptr && ldt < k) || ldp < (k + 3) / 4) return TERN_ERR_STRIDE;
  const uintptr_t esz = (w_dtype == TERN_F32) ? 4 : 2;
  if (!aligned(w, esz) || !aligned(s, 4)) return TERN_ERR_ALIGN;
  return from_hip(tern::launch_quantize(w, w_dtype == TERN_BF16, n, k, ldw, t, ldt, s, p, ldp,
                                        static_cast<hipStream_t>(stream)));
}

tern_status tern_pack(const int8_t* t, int64_t n, int64_t k, int64_t ldt, uint8_t* p, int64_t ldp,
                      void* stream) {
  if (n < 0 || k < 0) return TERN_ERR_SHAPE;
  if (n == 0 || k == 0) return TERN_OK;
  if (t == nullptr || p == nullptr) return TERN_ERR_NULL;
  if (ldt < k || ldp < (k + 3) / 4) return TERN_ERR_STRIDE;
  return from_hip(tern::launch_pack(t, n, k, ldt, p, ldp, static_cast<hipStream_t>(stream)));
}

tern_status tern_unpack(const uint8_t* p, int64_t n, int64_t k, int64_t ldp, int8_t* t,
                        int64_t ldt, void* stream) {
  if (n < 0 || k < 0) return TERN_ERR_SHAPE;
  if (n == 0 || k == 0) return TERN_OK;
  if (p == nullptr || t == nullptr) return TERN_ERR_NULL;
  if (ldp < (k + 3) / 4 || ldt < k) return TERN_ERR_STRIDE;
  return from_hip(tern::launch_unpack(p, n, k, ldp, t, ldt, static_cast<hipStream_t>(stream)));
}

namespace {

tern_status gemm_common(const void* x_bf16, int64_t m, int64_t k, int64_t ldx, const uint8_t* p,
                        int64_t n, int64_t ldp, const float* s, const float* bias,
                        int64_t act_from, void* y_bf16, int64_t ldy, void* stream) {
  if (m < 0 || n < 0 || k < 0 || m > kMaxInt || n > kMaxInt || k > kMaxInt - 63 || k % 64 != 0)
    return TERN_ERR_SHAPE;
  // The smallest tile is 64 x 128: the tile count must fit the grid.
  if (((m + 63) / 64) * ((n + 127) / 128) > kMaxInt) return TERN_ERR_SHAPE;
  if (m == 0 || n == 0) return TERN_OK;
  if (x_bf16 == nullptr || p == nullptr || s == nullptr || y_bf16 == nullptr) return TERN_ERR_NULL;
  if (ldx < k || ldp < k / 4 || ldy < n) return TERN_ERR_STRIDE;
  if (ldx > kGemmMaxLdx || ldp > kGemmMaxLdp || ldy > kMaxInt) return TERN_ERR_STRIDE;
  if (!aligned(x_bf16, 16) || ldx % 8 != 0 || !aligned(p, 16) || ldp % 16 != 0 ||
      !aligned(y_bf16, 2) || !aligned(s, 4) || !aligned(bias, 4))
    return TERN_ERR_ALIGN;
  return from_hip(tern::launch_gemm(static_cast<const uint16_t*>(x_bf16), m, k, ldx, p, n, ldp, s,
                                    bias, act_from, static_cast<uint16_t*>(y_bf16), ldy,
                                    static_cast<hipStream_t>(stream)));
}

}  // namespace

tern_status tern_gemm(const void* x_bf16, int64_t m, int64_t k, int64_t ldx, const uint8_t* p,
                      int64_t n, int64_t ldp, const float* s, void* y_bf16, int64_t ldy,
                      void* stream) {
  return gemm_common(x_bf16, m, k, ldx, p, n, ldp, s, nullptr, n, y_bf16, ldy, stream);
}

tern_status tern_gemm_ex(const void* x_bf16, int64_t m, int64_t k, int64_t ldx, const uint8_t* p,
                         int64_t n, int64_t ldp, const float* s, const float* bias, tern_act act,
                         int64_t act_from, void* y_bf16, int64_t ldy, void* stream) {
  if (act != TERN_ACT_NONE && act != TERN_ACT_GELU_TANH) return TERN_ERR_ARG;
  if (act == TERN_ACT_GELU_TANH && (act_from < 0 || act_from > n)) return TERN_ERR_ARG;
  return gemm_common(x_bf16, m, k, ldx, p, n, ldp, s, bias,
                     act == TERN_ACT_GELU_TANH ? act_from : n, y_bf16, ldy, stream);
}

tern_status tern_pack_transposed(const uint8_t* p, int64_t n, int64_t k, int64_t ldp, uint8_t* pt,
                                 int64_t ldpt, void* stream) {
  if (n < 0 || k < 0 || n > kMaxInt || k > kMaxInt) return TERN_ERR_SHAPE;
  if (n == 0 || k == 0) return TERN_OK;
  if (p == nullptr || pt == nullptr) return TERN_ERR_NULL;
  if (ldp < (k + 3) / 4 || ldpt < (n + 3) / 4) return TERN_ERR_STRIDE;
  return from_hip(
      tern::launch_pack_transposed(p, n, k, ldp, pt, ldpt, static_cast<hipStream_t>(stream)));
}

tern_status tern_gemm_dx(const void* dy_bf16, int64_t m, int64_t n, int64_t lddy,
                         const uint8_t* pt, int64_t k, int64_t ldpt, const float* s,
                         void* u_bf16, int64_t ldu, void* dx_bf16, int64_t lddx, void* stream) {
  // The product is the layer's GEMM with the roles renamed: u [m, n] is the
  // activation operand, pt (rows k, packed along n) the weights, n the
  // contraction and k the output width; unit scales.
  if (m < 0 || n < 0 || k < 0 || m > kMaxInt || k > kMaxInt || n > kMaxInt - 63 || n % 64 != 0)
    return TERN_ERR_SHAPE;
  if (((m + 63) / 64) * ((k + 127) / 128) > kMaxInt) return TERN_ERR_SHAPE;
  if (m == 0 || k == 0) return TERN_OK;
  // With n == 0 the gradient, the scales and the workspace are not read.
  if (pt == nullptr || dx_bf16 == nullptr ||
      (n > 0 && (dy_bf16 == nullptr || s == nullptr || u_bf16 == nullptr)))
    return TERN_ERR_NULL;
  if (lddy < n || ldu < n || ldpt < n / 4 || lddx < k) return TERN_ERR_STRIDE;
  if ((n > 0 && ldu > kGemmMaxLdx) || ldpt > kGemmMaxLdp || lddx > kMaxInt) return TERN_ERR_STRIDE;
  if (!aligned(pt, 16) || ldpt % 16 != 0 || !aligned(dx_bf16, 2)) return TERN_ERR_ALIGN;
  if (n > 0 && (!aligned(dy_bf16, 2) || !aligned(u_bf16, 16) || ldu % 8 != 0 || !aligned(s, 4)))
    return TERN_ERR_ALIGN;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  uint16_t* u = static_cast<uint16_t*>(u_bf16);
  if (n > 0) {
    const hipError_t e =
        tern::launch_scale_grad(static_cast<const uint16_t*>(dy_bf16), m, n, lddy, s, u, ldu, st);
    if (e != hipSuccess) return TERN_ERR_HIP;
  }
  return from_hip(tern::launch_gemm(u, m, n, ldu, pt, k, ldpt, nullptr, nullptr, k,
                                    static_cast<uint16_t*>(dx_bf16), lddx, st));
}

tern_status tern_gemm_dx_static(const void* dy_bf16, int64_t m, int64_t n, int64_t lddy,
                                const uint8_t* pt, int64_t k, int64_t ldpt, const float* s,
                                void* dx_bf16, int64_t lddx, void* stream) {
  // tern_gemm_dx with the scaled gradient in the library's device array
  // (row pitch n): the rules of tern_gemm_dx without u and ldu, and a bound
  // on m * n.
  static_assert(TERN_GEMM_DX_STATIC_MAX_ELEMS == tern::kStaticScratchElems, "header limit");
  if (m < 0 || n < 0 || k < 0 || m > kMaxInt || k > kMaxInt || n > kMaxInt - 63 || n % 64 != 0)
    return TERN_ERR_SHAPE;
  if (((m + 63) / 64) * ((k + 127) / 128) > kMaxInt) return TERN_ERR_SHAPE;
  if (n > 0 && m > TERN_GEMM_DX_STATIC_MAX_ELEMS / n) return TERN_ERR_SHAPE;
  if (m == 0 || k == 0) return TERN_OK;
  if (pt == nullptr || dx_bf16 == nullptr || (n > 0 && (dy_bf16 == nullptr || s == nullptr)))
    return TERN_ERR_NULL;
  if (lddy < n || ldpt < n / 4 || lddx < k) return TERN_ERR_STRIDE;
  if ((n > 0 && n > kGemmMaxLdx) || ldpt > kGemmMaxLdp || lddx > kMaxInt) return TERN_ERR_STRIDE;
  if (!aligned(pt, 16) || ldpt % 16 != 0 || !aligned(dx_bf16, 2)) return TERN_ERR_ALIGN;
  if (n > 0 && (!aligned(dy_bf16, 2) || !aligned(s, 4))) return TERN_ERR_ALIGN;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  uint16_t* u = nullptr;
  if (n > 0) {
    if (tern::static_scratch(st, &u) != hipSuccess) return TERN_ERR_HIP;
    // Every element of u [m, n] is written before the product reads it.
    const hipError_t e =
        tern::launch_scale_grad(static_cast<const uint16_t*>(dy_bf16), m, n, lddy, s, u, n, st);
    if (e != hipSuccess) return TERN_ERR_HIP;
  }
  return from_hip(tern::launch_gemm(u, m, n, n, pt, k, ldpt, nullptr, nullptr, k,
                                    static_cast<uint16_t*>(dx_bf16), lddx, st));
}

tern_status tern_gemm_dw(const void* dy_bf16, int64_t m, int64_t n, int64_t lddy,
                         const void* x_bf16, int64_t k, int64_t ldx, float* dw, int64_t lddw,
                         int accumulate, void* stream) {
  if (m < 0 || n < 0 || k < 0 || m > kMaxInt || n > kMaxInt || k > kMaxInt) return TERN_ERR_SHAPE;
  // The smallest tile is 128 x 128: the tile count must fit the grid.
  if (((n + 127) / 128) * ((k + 127) / 128) > kMaxInt) return TERN_ERR_SHAPE;
  if (n == 0 || k == 0) return TERN_OK;
  if (dw == nullptr || (m > 0 && (dy_bf16 == nullptr || x_bf16 == nullptr))) return TERN_ERR_NULL;
  if (lddw < k || (m > 0 && (lddy < n || ldx < k))) return TERN_ERR_STRIDE;
  if (lddw > kMaxInt) return TERN_ERR_STRIDE;
  // A stage's buffer resource spans the rest of the matrix from its first
  // token: its byte count must fit 32 bits.
  if (m > 0 && ((m - 1) * lddy + (n + 7) / 8 * 8 > kMaxInt || (m - 1) * ldx + (k + 7) / 8 * 8 > kMaxInt))
    return TERN_ERR_SHAPE;
  if (!aligned(dw, 4)) return TERN_ERR_ALIGN;
  if (m > 0 && (!aligned(dy_bf16, 16) || lddy % 8 != 0 || !aligned(x_bf16, 16) || ldx % 8 != 0))
    return TERN_ERR_ALIGN;
  return from_hip(tern::launch_gemm_dw(static_cast<const uint16_t*>(dy_bf16), m, n, lddy,
                                       static_cast<const uint16_t*>(x_bf16), k, ldx, dw, lddw,
                                       accumulate != 0, static_cast<hipStream_t>(stream)));
}

tern_status tern_quantize_act(const void* x_bf16, int64_t m, int64_t k, int64_t ldx, int8_t* q,
                              int64_t ldq, float* xs, void* stream) {
  if (m < 0 || k < 0 || m > kMaxInt || k > kMaxInt) return TERN_ERR_SHAPE;
  if (m == 0) return TERN_OK;
  if (xs == nullptr || (k > 0 && (x_bf16 == nullptr || q == nullptr))) return TERN_ERR_NULL;
  if (ldx < k || ldq < k) return TERN_ERR_STRIDE;
  if (!aligned(x_bf16, 2) || !aligned(xs, 4)) return TERN_ERR_ALIGN;
  return from_hip(tern::launch_quantize_act(static_cast<const uint16_t*>(x_bf16), m, k, ldx, q,
                                            ldq, xs, static_cast<hipStream_t>(stream)));
}

tern_status tern_pack_a8(const uint8_t* p, int64_t n, int64_t k, int64_t ldp, uint8_t* p8,
                         int64_t ldp8, void* stream) {
  if (n < 0 || k < 0 || n > kMaxInt || k > kMaxInt || k % 16 != 0) return TERN_ERR_SHAPE;
  if (n == 0 || k == 0) return TERN_OK;
  if (p == nullptr || p8 == nullptr) return TERN_ERR_NULL;
  if (ldp < k / 4 || ldp8 < k / 4) return TERN_ERR_STRIDE;
  if (!aligned(p, 4) || !aligned(p8, 4) || ldp % 4 != 0 || ldp8 % 4 != 0) return TERN_ERR_ALIGN;
  return from_hip(tern::launch_pack_a8(p, n, k, ldp, p8, ldp8, static_cast<hipStream_t>(stream)));
}

tern_status tern_gemm_a8(const int8_t* q, int64_t m, int64_t k, int64_t ldq, const float* xs,
                         const uint8_t* p8, int64_t n, int64_t ldp8, const float* s,
                         const float* bias, tern_act act, int64_t act_from, void* y_bf16,
                         int64_t ldy, void* stream) {
  if (act != TERN_ACT_NONE && act != TERN_ACT_GELU_TANH) return TERN_ERR_ARG;
  if (act == TERN_ACT_GELU_TANH && (act_from < 0 || act_from > n)) return TERN_ERR_ARG;
  // |sum| <= 127 * 64 * k < 2^31 for k <= 2^18.
  if (m < 0 || n < 0 || k < 0 || m > kMaxInt || n > kMaxInt || k > (int64_t(1) << 18) ||
      k % 128 != 0)
    return TERN_ERR_SHAPE;
  if (((m + 63) / 64) * ((n + 127) / 128) > kMaxInt) return TERN_ERR_SHAPE;
  if (m == 0 || n == 0) return TERN_OK;
  if (q == nullptr || xs == nullptr || p8 == nullptr || s == nullptr || y_bf16 == nullptr)
    return TERN_ERR_NULL;
  if (ldq < k || ldp8 < k / 4 || ldy < n) return TERN_ERR_STRIDE;
  if (ldq > kGemmMaxLdp || ldp8 > kGemmMaxLdp || ldy > kMaxInt) return TERN_ERR_STRIDE;
  if (!aligned(q, 16) || ldq % 16 != 0 || !aligned(p8, 16) || ldp8 % 16 != 0 ||
      !aligned(y_bf16, 2) || !aligned(xs, 4) || !aligned(s, 4) || !aligned(bias, 4))
    return TERN_ERR_ALIGN;
  return from_hip(tern::launch_gemm_a8(q, m, k, ldq, xs, p8, n, ldp8, s, bias,
                                       act == TERN_ACT_GELU_TANH ? act_from : n,
                                       static_cast<uint16_t*>(y_bf16), ldy,
                                       static_cast<hipStream_t>(stream)));
}

const char* tern_status_string(tern_status status) {
  switch (status) {
    case TERN_OK: return "TERN_OK: success";
    case TERN_ERR_NULL: return "TERN_ERR_NULL: a required pointer is NULL";
    case TERN_ERR_SHAPE: return "TERN_ERR_SHAPE: a size is negative or outside the supported range";
    case TERN_ERR_ALIGN: return "TERN_ERR_ALIGN: a pointer or leading dimension breaks an alignment rule";
    case TERN_ERR_STRIDE: return "TERN_ERR_STRIDE: a leading dimension is too short or too long";
    case TERN_ERR_DTYPE: return "TERN_ERR_DTYPE: unknown element type";
    case TERN_ERR_HIP: return "TERN_ERR_HIP: the HIP runtime rejected a launch";
    case TERN_ERR_ARG: return "TERN_ERR_ARG: an argument is outside its set of allowed values";
  }
  return "unknown tern_status";
}

}  // extern "C"
