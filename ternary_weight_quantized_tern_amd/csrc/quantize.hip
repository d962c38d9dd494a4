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
// codes.  Per weight: 4 (or 2) bytes read, 1 byte written, and about fifteen
// VALU instructions (the fixed-point term is formed with exact fp32 scaling
// and floors rather than 64-bit integer shifts).
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

// Adds q = floor(|a| * 2^(48 - E)) for the fp32 magnitude with bit pattern
// `abits` (|a| <= 2^(E+1), so q < 2^49) to a split accumulator: q = h * 2^32 +
// l with h < 2^17 and l < 2^32.  Every step is exact in fp32: the scaling by a
// power of two (a result below 1 may lose bits but floors to 0 either way),
// the floors of values below 2^49, and l = x - h * 2^32, a multiple of
// ulp(x) below 2^32.
__device__ inline void fixed_point_add(uint32_t abits, int E, uint32_t& acc_hi,
                                       unsigned long long& acc_lo) {
  const float x = __builtin_floorf(__builtin_ldexpf(__uint_as_float(abits), 48 - E));
  const float h = __builtin_floorf(x * 0x1p-32f);
  const float l = __builtin_fmaf(h, -0x1p32f, x);
  acc_hi += static_cast<uint32_t>(h);
  acc_lo += static_cast<uint32_t>(l);
}

// Code of one weight (fp32 bit pattern b) against the row scale s.
__device__ inline int8_t ternary_code(uint32_t b, float s) {
  const float mag = __uint_as_float(b & 0x7FFFFFFFu);
  return (2.0f * mag > s) ? ((b >> 31) ? int8_t(-1) : int8_t(1)) : int8_t(0);
}

// E = floor(log2(m)) for the fp32 magnitude bits m != 0 (normal or subnormal).
__device__ inline int floor_log2_bits(uint32_t m) {
  const uint32_t ef = m >> 23;
  return ef != 0 ? static_cast<int>(ef) - 127 : (31 - __clz(static_cast<int>(m))) - 149;
}

// s = fp32(Q * 2^(E - 48) / k), each step rounded to nearest.
__device__ inline float scale_of(unsigned long long q, int E, int64_t k) {
  return static_cast<float>(ldexp(static_cast<double>(q), E - 48) / static_cast<double>(k));
}

// With PACK, the codes also go out packed four to a byte (weight k in bits
// 2(k%4) .. 2(k%4)+1 of byte k/4 of row n of p, fields past k zero), exactly
// as the pack kernel writes them, and t may be null (codes not written).
template <typename TIn, int VEC, int CAP, bool PACK>
__global__ __launch_bounds__(kThreads) void quantize_rows(const TIn* __restrict__ w, int64_t k,
                                                          int64_t ldw, int8_t* __restrict__ t,
                                                          int64_t ldt, float* __restrict__ s,
                                                          uint8_t* __restrict__ p, int64_t ldp) {
  constexpr int kChunks = CAP / VEC;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const TIn* wr = w + row * ldw;
  const bool write_t = !PACK || t != nullptr;
  int8_t* tr = write_t ? t + row * ldt : nullptr;
  uint8_t* pr = PACK ? p + row * ldp : nullptr;
  const int64_t nbytes = (k + 3) / 4;

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
    const int E = floor_log2_bits(amax);
    uint32_t q_hi = 0;           // < 2^17 * CAP
    unsigned long long q_lo = 0;  // < 2^32 * CAP
#pragma unroll
    for (int i = 0; i < CAP; ++i) fixed_point_add(a[i] & 0x7FFFFFFFu, E, q_hi, q_lo);
    const unsigned long long q = wave_sum_u64((static_cast<unsigned long long>(q_hi) << 32) + q_lo);
    if (lane == 0) red_sum[wave] = q;
    __syncthreads();
    unsigned long long total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) total += red_sum[i];
    scale = scale_of(total, E, k);
  }
  if (tid == 0) s[row] = scale;

  // T = sign(w) where 2|w| > s, else 0.  The comparison is exact in fp32:
  // doubling is exact (a magnitude of 2^127 or more doubles to +inf, which
  // exceeds every finite s, as 2|w| does).  An all-zero row has s = 0 and
  // every |w| = 0, so it also yields T = 0.
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int64_t e0 = (static_cast<int64_t>(c) * kThreads + tid) * VEC;
    int8_t code[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) code[v] = ternary_code(a[c * VEC + v], scale);
    if constexpr (PACK) {
      if constexpr (VEC == 1) {
        // Four consecutive weights belong to four neighbouring lanes (e0 % 4
        // is tid % 4): OR their fields together, the first lane writes.
        uint32_t b = (static_cast<uint32_t>(code[0]) & 3u) << (2 * (e0 & 3));
        b |= __shfl_xor(b, 1, 64);
        b |= __shfl_xor(b, 2, 64);
        if ((e0 & 3) == 0 && e0 / 4 < nbytes) pr[e0 / 4] = static_cast<uint8_t>(b);
      } else {
#pragma unroll
        for (int q = 0; q < VEC / 4; ++q) {
          uint32_t b = 0;
#pragma unroll
          for (int v = 0; v < 4; ++v) b |= (static_cast<uint32_t>(code[4 * q + v]) & 3u) << (2 * v);
          if (e0 / 4 + q < nbytes) pr[e0 / 4 + q] = static_cast<uint8_t>(b);
        }
      }
      if (!write_t) continue;
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


template <typename TIn, int VEC, bool PACK>
hipError_t launch_cap(const TIn* w, int64_t n, int64_t k, int64_t ldw, int8_t* t, int64_t ldt,
                      float* s, uint8_t* p, int64_t ldp, hipStream_t stream) {
  const int64_t per_thread = (k + kThreads - 1) / kThreads;
  dim3 grid(static_cast<unsigned>(n)), block(kThreads);
#define TERN_Q_LAUNCH(CAP)                                                                   \
  if (per_thread <= CAP) {                                                                   \
    hipLaunchKernelGGL((quantize_rows<TIn, VEC, (CAP < VEC ? VEC : CAP), PACK>), grid, block, \
                       0, stream, w, k, ldw, t, ldt, s, p, ldp);                             \
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

template <bool PACK>
hipError_t launch_variant(const void* w, bool w_is_bf16, int64_t n, int64_t k, int64_t ldw,
                          int8_t* t, int64_t ldt, float* s, uint8_t* p, int64_t ldp,
                          hipStream_t stream) {
  // Vector loads (and vector stores of the codes) where the rows allow them.
  const bool t_vec4 = t == nullptr || (aligned(t, 4) && ldt % 4 == 0);
  const bool t_vec8 = t == nullptr || (aligned(t, 8) && ldt % 8 == 0);
  if (!w_is_bf16) {
    const float* wf = static_cast<const float*>(w);
    if (aligned(w, 16) && ldw % 4 == 0 && t_vec4)
      return launch_cap<float, 4, PACK>(wf, n, k, ldw, t, ldt, s, p, ldp, stream);
    return launch_cap<float, 1, PACK>(wf, n, k, ldw, t, ldt, s, p, ldp, stream);
  }
  const uint16_t* wb = static_cast<const uint16_t*>(w);
  if (aligned(w, 16) && ldw % 8 == 0 && t_vec8)
    return launch_cap<uint16_t, 8, PACK>(wb, n, k, ldw, t, ldt, s, p, ldp, stream);
  return launch_cap<uint16_t, 1, PACK>(wb, n, k, ldw, t, ldt, s, p, ldp, stream);
}

}  // namespace

hipError_t launch_quantize(const void* w, bool w_is_bf16, int64_t n, int64_t k, int64_t ldw,
                           int8_t* t, int64_t ldt, float* s, uint8_t* p, int64_t ldp,
                           hipStream_t stream) {
  if (p != nullptr) return launch_variant<true>(w, w_is_bf16, n, k, ldw, t, ldt, s, p, ldp, stream);
  return launch_variant<false>(w, w_is_bf16, n, k, ldw, t, ldt, s, nullptr, 0, stream);
}

}  // namespace tern
