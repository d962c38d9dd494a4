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
// in cache).  A thread converts groups of 8 consecutive elements of a row
// with 16-byte loads and stores where the pointers and pitches allow it, else
// one at a time; a grid-stride loop covers any m x n.
#include <mutex>

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

// Each thread converts G groups of 8 elements, grid-stride apart, with all G
// loads issued before the first conversion (more bytes in flight per thread).
template <int G>
__global__ __launch_bounds__(kThreads) void scale_grad_kernel(const uint16_t* __restrict__ dy,
                                                              int64_t m, int64_t n, int64_t lddy,
                                                              const float* __restrict__ s,
                                                              uint16_t* __restrict__ u,
                                                              int64_t ldu, bool vec) {
  const int64_t groups = (n + 7) / 8;  // 8 elements per group
  const int64_t total = m * groups;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; base < total;
       base += stride * G) {
    uint4 v[G];
    int64_t row[G], c0[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int64_t idx = base + g * stride;
      row[g] = idx / groups;
      c0[g] = (idx - row[g] * groups) * 8;
      if (idx < total && vec && c0[g] + 8 <= n)
        v[g] = *reinterpret_cast<const uint4*>(dy + row[g] * lddy + c0[g]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (base + g * stride >= total) continue;
      const uint16_t* src = dy + row[g] * lddy + c0[g];
      uint16_t* dst = u + row[g] * ldu + c0[g];
      if (vec && c0[g] + 8 <= n) {
        const float4 s0 = *reinterpret_cast<const float4*>(s + c0[g]);
        const float4 s1 = *reinterpret_cast<const float4*>(s + c0[g] + 4);
        uint4 o;
        o.x = to_bf16x2(bf16_to_f32(v[g].x & 0xFFFFu) * s0.x, bf16_to_f32(v[g].x >> 16) * s0.y);
        o.y = to_bf16x2(bf16_to_f32(v[g].y & 0xFFFFu) * s0.z, bf16_to_f32(v[g].y >> 16) * s0.w);
        o.z = to_bf16x2(bf16_to_f32(v[g].z & 0xFFFFu) * s1.x, bf16_to_f32(v[g].z >> 16) * s1.y);
        o.w = to_bf16x2(bf16_to_f32(v[g].w & 0xFFFFu) * s1.z, bf16_to_f32(v[g].w >> 16) * s1.w);
        *reinterpret_cast<uint4*>(dst) = o;
      } else {
        for (int e = 0; e < 8 && c0[g] + e < n; ++e)
          dst[e] = static_cast<uint16_t>(to_bf16x2(bf16_to_f32(src[e]) * s[c0[g] + e], 0.0f) &
                                         0xFFFFu);
      }
    }
  }
}

// The device array behind tern_gemm_dx_static: the scaled gradient u of one
// call, for callers that cannot allocate.  Every GPU that runs the library
// holds its own copy (kStaticScratchElems bf16 values) from the module's load
// until the process ends.  In host code `scratch` names a host-side stand-in:
// its device address on a GPU comes from hipGetSymbolAddress, taken once per
// device and kept in g_scratch_ptr.
__device__ __align__(256) uint16_t scratch[kStaticScratchElems];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(hipStream_t stream, uint16_t** ptr) {
  int dev = 0;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    // The symbol's address is per device: look it up with that device current.
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = static_cast<uint16_t*>(g_scratch_ptr[dev]);
  return hipSuccess;
}

hipError_t launch_scale_grad(const uint16_t* dy, int64_t m, int64_t n, int64_t lddy,
                             const float* s, uint16_t* u, int64_t ldu, hipStream_t stream) {
  const bool vec = reinterpret_cast<uintptr_t>(dy) % 16 == 0 && lddy % 8 == 0 &&
                   reinterpret_cast<uintptr_t>(u) % 16 == 0 && ldu % 8 == 0 &&
                   reinterpret_cast<uintptr_t>(s) % 16 == 0;
  // Two groups per thread: 5 % faster than one on the DiT up-projection's
  // backward (2048 x 4608), the same on the FLUX shapes.
  constexpr int kGroups = 2;
  int64_t blocks = (m * ((n + 7) / 8) + kThreads * kGroups - 1) / (kThreads * kGroups);
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(scale_grad_kernel<kGroups>, dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), 0, stream, dy, m, n, lddy, s, u, ldu, vec);
  return hipGetLastError();
}

}  // namespace tern
