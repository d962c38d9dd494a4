// Absmean ternarization with one scale per output channel.
//
// "1.58-bit FLUX" (arXiv 2412.18653), section 1: the weights of every linear
// layer are restricted to {+1, 0, -1} as in BitNet b1.58.  The pages give no
// formula; the rule implemented is s_n = mean_k |w_nk| and
// T_nk = clip(round(w_nk / s_n), -1, 1) with ties to even, where the mean is
// taken in 64-bit fixed point so that it is independent of the summation
// order (the full definition is in include/ternary.h).
//
// One workgroup of 256 threads owns one row.  The row is read from HBM once
// and kept in registers (up to 128 elements per thread, K <= 32768); the two
// reductions (max of |w|, then the integer sum) are wave-level butterflies
// followed by a 4-entry LDS combine; then each thread writes its ternary
// codes.  The work is HBM-bound: 4 (or 2) bytes read and 1 byte written per
// weight.
#include "internal.h"

namespace tern {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ inline uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

__device__ inline unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// fp32 bit pattern of element e of one row (bf16 widened exactly).
template <typename TIn>
__device__ inline uint32_t bits_of(TIn v);
template <>
__device__ inline uint32_t bits_of<float>(float v) {
  return __float_as_uint(v);
}
template <>
__device__ inline uint32_t bits_of<uint16_t>(uint16_t v) {
  return static_cast<uint32_t>(v) << 16;
}

// floor(|a| * 2^(48 - E)) for the fp32 magnitude with bit pattern `abits`,
// computed on the integer significand: |a| = m * 2^(ef - 150), ef >= 1.
__device__ inline unsigned long long fixed_point_term(uint32_t abits, int E) {
  uint32_t ef = abits >> 23;
  uint32_t m = abits & 0x7FFFFFu;
  if (ef != 0) {
    m |= 0x800000u;
  } else {
    ef = 1;
  }
  int sh = static_cast<int>(ef) - 102 - E;  // <= 25 because |a| <= 2^(E+1)
  if (sh >= 0) return static_cast<unsigned long long>(m) << sh;
  if (sh > -32) return static_cast<unsigned long long>(m >> (-sh));
  return 0ull;
}

template <typename TIn, int VEC, int CAP>
__global__ __launch_bounds__(kThreads) void quantize_rows(const TIn* __restrict__ w, int64_t k,
                                                          int64_t ldw, int8_t* __restrict__ t,
                                                          int64_t ldt, float* __restrict__ s) {
  constexpr int kChunks = CAP / VEC;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const TIn* wr = w + row * ldw;
  int8_t* tr = t + row * ldt;

  uint32_t a[CAP];  // fp32 bit patterns, sign included
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int64_t e0 = (static_cast<int64_t>(c) * kThreads + tid) * VEC;
    if constexpr (VEC > 1) {
      if (e0 + VEC <= k) {
        if constexpr (sizeof(TIn) == 4) {
          float4 v = *reinterpret_cast<const float4*>(wr + e0);
          a[c * VEC + 0] = __float_as_uint(v.x);
          a[c * VEC + 1] = __float_as_uint(v.y);
          a[c * VEC + 2] = __float_as_uint(v.z);
          a[c * VEC + 3] = __float_as_uint(v.w);
        } else {
          uint4 v = *reinterpret_cast<const uint4*>(wr + e0);
          const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            a[c * VEC + 2 * j] = d[j] << 16;
            a[c * VEC + 2 * j + 1] = d[j] & 0xFFFF0000u;
          }
        }
        continue;
      }
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) a[c * VEC + v] = (e0 + v < k) ? bits_of<TIn>(wr[e0 + v]) : 0u;
  }

  __shared__ uint32_t red_max[kWaves];
  __shared__ unsigned long long red_sum[kWaves];
  const int wave = tid >> 6;
  const int lane = tid & 63;

  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < CAP; ++i) {
    uint32_t ab = a[i] & 0x7FFFFFFFu;
    amax = ab > amax ? ab : amax;
  }
  amax = wave_max_u32(amax);
  if (lane == 0) red_max[wave] = amax;
  __syncthreads();
  amax = red_max[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) amax = red_max[i] > amax ? red_max[i] : amax;

  float scale = 0.0f;
  if (amax != 0u) {
    // E = floor(log2(max |w|)), exact for normal and subnormal maxima.
    const uint32_t ef = amax >> 23;
    const int E = ef != 0 ? static_cast<int>(ef) - 127 : (31 - __clz(static_cast<int>(amax))) - 149;
    unsigned long long q = 0;
#pragma unroll
    for (int i = 0; i < CAP; ++i) q += fixed_point_term(a[i] & 0x7FFFFFFFu, E);
    q = wave_sum_u64(q);
    if (lane == 0) red_sum[wave] = q;
    __syncthreads();
    unsigned long long total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) total += red_sum[i];
    const double mean = ldexp(static_cast<double>(total), E - 48) / static_cast<double>(k);
    scale = static_cast<float>(mean);
  }
  if (tid == 0) s[row] = scale;

  // T = sign(w) where 2|w| > s (exact in double), else 0.  An all-zero row has
  // s = 0 and every |w| = 0, so it also yields T = 0.
  const double sd = static_cast<double>(scale);
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int64_t e0 = (static_cast<int64_t>(c) * kThreads + tid) * VEC;
    int8_t code[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const uint32_t b = a[c * VEC + v];
      const double mag = static_cast<double>(__uint_as_float(b & 0x7FFFFFFFu));
      const bool nz = 2.0 * mag > sd && amax != 0u;
      code[v] = nz ? ((b >> 31) ? int8_t(-1) : int8_t(1)) : int8_t(0);
    }
    if constexpr (VEC == 4) {
      if (e0 + 4 <= k) {
        uint32_t packed = (uint32_t(uint8_t(code[0]))) | (uint32_t(uint8_t(code[1])) << 8) |
                          (uint32_t(uint8_t(code[2])) << 16) | (uint32_t(uint8_t(code[3])) << 24);
        *reinterpret_cast<uint32_t*>(tr + e0) = packed;
        continue;
      }
    } else if constexpr (VEC == 8) {
      if (e0 + 8 <= k) {
        uint2 packed;
        packed.x = (uint32_t(uint8_t(code[0]))) | (uint32_t(uint8_t(code[1])) << 8) |
                   (uint32_t(uint8_t(code[2])) << 16) | (uint32_t(uint8_t(code[3])) << 24);
        packed.y = (uint32_t(uint8_t(code[4]))) | (uint32_t(uint8_t(code[5])) << 8) |
                   (uint32_t(uint8_t(code[6])) << 16) | (uint32_t(uint8_t(code[7])) << 24);
        *reinterpret_cast<uint2*>(tr + e0) = packed;
        continue;
      }
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v)
      if (e0 + v < k) tr[e0 + v] = code[v];
  }
}

template <typename TIn, int VEC>
hipError_t launch_cap(const TIn* w, int64_t n, int64_t k, int64_t ldw, int8_t* t, int64_t ldt,
                      float* s, hipStream_t stream) {
  const int64_t per_thread = (k + kThreads - 1) / kThreads;
  dim3 grid(static_cast<unsigned>(n)), block(kThreads);
#define TERN_Q_LAUNCH(CAP)                                                                   \
  if (per_thread <= CAP) {                                                                   \
    hipLaunchKernelGGL((quantize_rows<TIn, VEC, (CAP < VEC ? VEC : CAP)>), grid, block, 0, \
                       stream, w, k, ldw, t, ldt, s);                                        \
    return hipGetLastError();                                                                \
  }
  TERN_Q_LAUNCH(8)
  TERN_Q_LAUNCH(16)
  TERN_Q_LAUNCH(32)
  TERN_Q_LAUNCH(64)
  TERN_Q_LAUNCH(128)
#undef TERN_Q_LAUNCH
  return hipErrorInvalidValue;  // k > 32768 is rejected before this point
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

hipError_t launch_quantize(const void* w, bool w_is_bf16, int64_t n, int64_t k, int64_t ldw,
                           int8_t* t, int64_t ldt, float* s, hipStream_t stream) {
  if (!w_is_bf16) {
    const float* wf = static_cast<const float*>(w);
    if (aligned(w, 16) && ldw % 4 == 0 && aligned(t, 4) && ldt % 4 == 0)
      return launch_cap<float, 4>(wf, n, k, ldw, t, ldt, s, stream);
    return launch_cap<float, 1>(wf, n, k, ldw, t, ldt, s, stream);
  }
  const uint16_t* wb = static_cast<const uint16_t*>(w);
  if (aligned(w, 16) && ldw % 8 == 0 && aligned(t, 8) && ldt % 8 == 0)
    return launch_cap<uint16_t, 8>(wb, n, k, ldw, t, ldt, s, stream);
  return launch_cap<uint16_t, 1>(wb, n, k, ldw, t, ldt, s, stream);
}

}  // namespace tern
