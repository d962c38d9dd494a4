// The scaled output gradient of the ternary layer, the operand of its input
// gradient.
//
// "TerDiT: Ternary Diffusion Models with Transformers" (abstract) trains
// ternary DiT weights in the loop (quantization-aware training); the pages
// give no formula.  For Y = (X . T^T) (.) s the input gradient is
// dX = (dY (.) s) . T; this kernel forms u = bf16(fp32(dY) * s_n) (one
// single-precision product, one round-to-nearest-even conversion), the bf16
// operand that the ternary GEMM then contracts over n with the codes packed
// along n.
//
// HBM-bound stream: 2 bytes read and 2 written per element (the scales stay
// in cache).  One thread converts 8 consecutive elements of a row with 16-byte
// loads and stores where the pointers and pitches allow it, else one at a
// time; a grid-stride loop covers any m x n.
#include "internal.h"

namespace tern {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kMaxBlocks = 256 * 64;

__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Two floats to two bf16 (round to nearest even) in one 32-bit word, low first.
__device__ inline uint32_t to_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__global__ __launch_bounds__(kThreads) void scale_grad_kernel(const uint16_t* __restrict__ dy,
                                                              int64_t m, int64_t n, int64_t lddy,
                                                              const float* __restrict__ s,
                                                              uint16_t* __restrict__ u,
                                                              int64_t ldu, bool vec) {
  const int64_t groups = (n + 7) / 8;  // 8 elements per group
  const int64_t total = m * groups;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int64_t row = idx / groups;
    const int64_t c0 = (idx - row * groups) * 8;
    const uint16_t* src = dy + row * lddy + c0;
    uint16_t* dst = u + row * ldu + c0;
    if (vec && c0 + 8 <= n) {
      const uint4 v = *reinterpret_cast<const uint4*>(src);
      const float4 s0 = *reinterpret_cast<const float4*>(s + c0);
      const float4 s1 = *reinterpret_cast<const float4*>(s + c0 + 4);
      uint4 o;
      o.x = to_bf16x2(bf16_to_f32(v.x & 0xFFFFu) * s0.x, bf16_to_f32(v.x >> 16) * s0.y);
      o.y = to_bf16x2(bf16_to_f32(v.y & 0xFFFFu) * s0.z, bf16_to_f32(v.y >> 16) * s0.w);
      o.z = to_bf16x2(bf16_to_f32(v.z & 0xFFFFu) * s1.x, bf16_to_f32(v.z >> 16) * s1.y);
      o.w = to_bf16x2(bf16_to_f32(v.w & 0xFFFFu) * s1.z, bf16_to_f32(v.w >> 16) * s1.w);
      *reinterpret_cast<uint4*>(dst) = o;
    } else {
      for (int e = 0; e < 8 && c0 + e < n; ++e)
        dst[e] = static_cast<uint16_t>(to_bf16x2(bf16_to_f32(src[e]) * s[c0 + e], 0.0f) & 0xFFFFu);
    }
  }
}

}  // namespace

hipError_t launch_scale_grad(const uint16_t* dy, int64_t m, int64_t n, int64_t lddy,
                             const float* s, uint16_t* u, int64_t ldu, hipStream_t stream) {
  const bool vec = reinterpret_cast<uintptr_t>(dy) % 16 == 0 && lddy % 8 == 0 &&
                   reinterpret_cast<uintptr_t>(u) % 16 == 0 && ldu % 8 == 0 &&
                   reinterpret_cast<uintptr_t>(s) % 16 == 0;
  int64_t blocks = (m * ((n + 7) / 8) + kThreads - 1) / kThreads;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(scale_grad_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     stream, dy, m, n, lddy, s, u, ldu, vec);
  return hipGetLastError();
}

}  // namespace tern
