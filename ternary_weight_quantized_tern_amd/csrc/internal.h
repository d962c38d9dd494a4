// Internal declarations of libternary: kernel launchers called by the C-ABI
// layer (api.hip) after it has validated every argument.  Not installed and
// not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tern {

// Launch geometry and the ld / alignment facts the launchers rely on are
// established by the caller (api.hip); each launcher returns the HIP status of
// its launch.
// p == nullptr: codes to t only.  Otherwise the codes also go to p packed
// (as launch_pack writes them), and t may be nullptr.
hipError_t launch_quantize(const void* w, bool w_is_bf16, int64_t n, int64_t k, int64_t ldw,
                           int8_t* t, int64_t ldt, float* s, uint8_t* p, int64_t ldp,
                           hipStream_t stream);

hipError_t launch_pack(const int8_t* t, int64_t n, int64_t k, int64_t ldt, uint8_t* p,
                       int64_t ldp, hipStream_t stream);

hipError_t launch_unpack(const uint8_t* p, int64_t n, int64_t k, int64_t ldp, int8_t* t,
                         int64_t ldt, hipStream_t stream);

// s: [n], or nullptr for unit scales (the input-gradient product); bias:
// nullptr or [n]; act_from in [0, n]: the tanh-form GELU is applied to
// columns >= act_from (act_from == n: no activation).
hipError_t launch_gemm(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const uint8_t* p,
                       int64_t n, int64_t ldp, const float* s, const float* bias,
                       int64_t act_from, uint16_t* y, int64_t ldy, hipStream_t stream);

// Layers with about one 64 x 144 output tile per CU and k >= 1024: the
// K-split kernel (called by launch_gemm for m > 32).
bool gemm_ksplit_fits(int64_t m, int64_t k, int64_t n);
hipError_t launch_gemm_ksplit(const uint16_t* x, int64_t m, int64_t k, int64_t ldx,
                              const uint8_t* p, int64_t n, int64_t ldp, const float* s,
                              const float* bias, int64_t act_from, uint16_t* y, int64_t ldy,
                              hipStream_t stream);

// m <= 32 (called by launch_gemm).
hipError_t launch_gemm_small(const uint16_t* x, int64_t m, int64_t k, int64_t ldx,
                             const uint8_t* p, int64_t n, int64_t ldp, const float* s,
                             const float* bias, int64_t act_from, uint16_t* y, int64_t ldy,
                             hipStream_t stream);

// Codes of p (rows n, packed along k) packed along n into pt (rows k).
hipError_t launch_pack_transposed(const uint8_t* p, int64_t n, int64_t k, int64_t ldp,
                                  uint8_t* pt, int64_t ldpt, hipStream_t stream);

// u = bf16(fp32(dy) * s[col]) for an m x n bf16 matrix.
hipError_t launch_scale_grad(const uint16_t* dy, int64_t m, int64_t n, int64_t lddy,
                             const float* s, uint16_t* u, int64_t ldu, hipStream_t stream);

// dw[n][k] = (accumulate ? dw : 0) + sum_m dy[m][n] * x[m][k], fp32 dw; dy
// and x 16-byte aligned with ld % 8 == 0, (m - 1) * ld + width < 2^31.
hipError_t launch_gemm_dw(const uint16_t* dy, int64_t m, int64_t n, int64_t lddy,
                          const uint16_t* x, int64_t k, int64_t ldx, float* dw, int64_t lddw,
                          bool accumulate, hipStream_t stream);

// Size of the per-device array that tern_gemm_dx_static uses for the scaled
// gradient (bf16 elements; 128 MiB).
inline constexpr int64_t kStaticScratchElems = int64_t(1) << 26;

// The device address of that array on the device of `stream` (the current
// device for the null stream), looked up once per device.
hipError_t static_scratch(hipStream_t stream, uint16_t** ptr);

// m <= 32 with int8 activations (called by launch_gemm_a8).
hipError_t launch_gemm_small_a8(const int8_t* q, int64_t m, int64_t k, int64_t ldq,
                                const float* xs, const uint8_t* p8, int64_t n, int64_t ldp8,
                                const float* s, const float* bias, int64_t act_from, uint16_t* y,
                                int64_t ldy, hipStream_t stream);

// Per-token int8 activations: q = rint(x * (127 / max|x|)), xs = max|x| / 127.
hipError_t launch_quantize_act(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, int8_t* q,
                               int64_t ldq, float* xs, hipStream_t stream);

// Codes of p (k % 16 == 0) in the field-transposed packing of the int8 GEMM.
hipError_t launch_pack_a8(const uint8_t* p, int64_t n, int64_t k, int64_t ldp, uint8_t* p8,
                          int64_t ldp8, hipStream_t stream);

// y = bf16(f(s[n] * xs[m] * (q . T^T) + bias)), k % 128 == 0, weights in the
// field-transposed packing; bias and act_from as for launch_gemm.
hipError_t launch_gemm_a8(const int8_t* q, int64_t m, int64_t k, int64_t ldq, const float* xs,
                          const uint8_t* p8, int64_t n, int64_t ldp8, const float* s,
                          const float* bias, int64_t act_from, uint16_t* y, int64_t ldy,
                          hipStream_t stream);

}  // namespace tern
