// Absmean ternarization with one scale per output channel.
//
// "1.58-bit FLUX" (arXiv 2412.18653), section 1: the weights of every linear
// layer are restricted to {+1, 0, -1} as in BitNet b1.58.  The pages give no
// formula; the rule implemented is s_n = mean_k |w_nk| and
// T_nk = clip(round(w_nk / s_n), -1, 1) with ties to even, where the mean is
// taken in 64-bit fixed point so that it is independent of the summation
// order (the full definition is in include/ternary.h).
//
// A row is owned by R = 1, 2 or 4 waves of a 256-thread workgroup (4, 2 or 1
// rows per workgroup).  The row is read from HBM once and kept in registers;
// the two reductions (max |w|, then the integer sum) are wave butterflies,
// combined across the row's waves through LDS when R > 1; then the codes are
// written, as int8 and/or packed four to a byte.  Per weight: 4 (or 2) bytes
// read, 1 byte (and/or 1/4 byte) written, and about fourteen VALU instructions
// (per-row reductions and addressing included):
//  - max |w| as the larger of the signed and the unsigned maximum of the bit
//    patterns (one 3-way max per two weights each);
//  - the fixed-point term floor(|w| * 2^(48 - E)) is an exact fp32 scaling
//    and floor, summed in fp64 in groups of 16 (every partial sum is an
//    integer below 2^53, so the fp64 additions are exact and the group sums
//    are converted to uint64 without loss);
//  - the ternary decision 2|w| > s is taken as |w| > h with h = s/2 rounded
//    toward zero, which is the same predicate for every float |w|, and the
//    sign comes from a median-of-three clamp of the bit pattern to [-1, 1];
//  - four codes are gathered into one 32-bit word with byte permutes, and
//    their 2-bit fields into one byte with a 4-way byte dot product.
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

// fp32 bit pattern of one element (bf16 widened exactly).
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

// floor(|a| * 2^sh) for the fp32 element with bit pattern `b`, where
// |a| < 2^(49 - sh): exact in fp32 (scaling by a power of two loses bits only
// below 1, where the floor is 0 either way; the floor of a value below 2^49
// is exact), returned as fp64 (exact).
__device__ inline double fixed_point_term(uint32_t b, int sh) {
  return static_cast<double>(
      __builtin_floorf(__builtin_ldexpf(__builtin_fabsf(__uint_as_float(b)), sh)));
}

// An fp64 holding an integer in [0, 2^53) as uint64 (both conversions exact).
__device__ inline unsigned long long u64_of(double v) {
  const double hi = __builtin_floor(v * 0x1p-32);
  const double lo = __builtin_fma(hi, -0x1p32, v);
  return (static_cast<unsigned long long>(static_cast<uint32_t>(hi)) << 32) |
         static_cast<uint32_t>(lo);
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

// h = s/2 rounded toward zero, for finite s >= 0.  For every float x >= 0,
// x > h exactly when 2x > s: if s/2 is a float, h equals it; otherwise h and
// the next float bracket s/2, and a float above s/2 is at least the next
// float.  Halving subtracts one from the exponent field when that leaves a
// normal number; below, the magnitude bits shift right by one (truncating).
__device__ inline float half_toward_zero(float s) {
  const uint32_t b = __float_as_uint(s);
  return __uint_as_float(b >= 0x01000000u ? b - 0x00800000u : b >> 1);
}

// Code byte of one weight: 0x01, 0xFF or 0x00 in the low byte (+1, -1, 0).
// The clamp of the bit pattern, read as int32, to [-1, 1] is the sign of every
// nonzero float (+0 clamps to 0, and |w| > h is false for it).
__device__ inline uint32_t code_of(uint32_t b, float h) {
  int32_t sgn;
  asm("v_med3_i32 %0, %1, -1, 1" : "=v"(sgn) : "v"(b));
  return (__builtin_fabsf(__uint_as_float(b)) > h) ? static_cast<uint32_t>(sgn) : 0u;
}

// Low bytes of four codes as one little-endian word.
__device__ inline uint32_t gather4(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
  const uint32_t lo = __builtin_amdgcn_perm(c1, c0, 0x0c0c0400u);  // c0.b0, c1.b0, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm(c3, c2, 0x04000c0cu);  // 0, 0, c2.b0, c3.b0
  return lo | hi;
}

// Four code bytes -> their 2-bit fields in one byte, weight j in bits 2j, 2j+1.
__device__ inline uint32_t pack4(uint32_t word) {
  return __builtin_amdgcn_udot4(word & 0x03030303u, 0x40100401u, 0u, false);
}

// One row per group of G = 64 * R threads (R = 1, 2, 4: four, two or one
// rows per workgroup).  Each thread holds CAP elements, CAP / VEC chunks of
// VEC consecutive elements; chunk c of thread g starts at (c * G + g) * VEC.
// t == nullptr skips the int8 codes, p == nullptr the packed bytes.
template <typename TIn, int VEC, int CAP, int R>
__global__ __launch_bounds__(kThreads) void quantize_rows(const TIn* __restrict__ w, int64_t n,
                                                          int k, int64_t ldw,
                                                          int8_t* __restrict__ t, int64_t ldt,
                                                          float* __restrict__ s,
                                                          uint8_t* __restrict__ p, int64_t ldp) {
  static_assert(R == 1 || R == 2 || R == 4, "a row is one, two or four waves");
  static_assert(CAP % VEC == 0 && (VEC == 1 || VEC % 4 == 0), "chunking");
  constexpr int G = 64 * R;
  constexpr int kRowsPerBlock = kWaves / R;
  constexpr int kChunks = CAP / VEC;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int grp = wave / R;  // row of this thread within the workgroup
  const int g = tid - grp * G;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + grp;
  if (R == 1 && row >= n) return;  // no barrier below when R == 1
  // With R > 1 every wave reaches the barriers; a group past the last row
  // reads the last row again and writes nothing.
  const bool valid = row < n;
  const int64_t row_in = valid ? row : n - 1;
  const TIn* wr = w + row_in * ldw;
  int8_t* tr = (t != nullptr && valid) ? t + row * ldt : nullptr;
  uint8_t* pr = (p != nullptr && valid) ? p + row * ldp : nullptr;
  const int nbytes = (k + 3) / 4;
  // Chunks 0 .. nfull-1 lie inside the row for every thread (no checks).
  const int nfull = k / (G * VEC);

  uint32_t a[CAP];  // fp32 bit patterns, sign included; zero past the row
  auto load_vec = [&](int c, int e0) {
    if constexpr (sizeof(TIn) == 4) {
      const float4 v = *reinterpret_cast<const float4*>(wr + e0);
      a[c * VEC + 0] = __float_as_uint(v.x);
      a[c * VEC + 1] = __float_as_uint(v.y);
      a[c * VEC + 2] = __float_as_uint(v.z);
      a[c * VEC + 3] = __float_as_uint(v.w);
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(wr + e0);
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[c * VEC + 2 * j] = d[j] << 16;
        a[c * VEC + 2 * j + 1] = d[j] & 0xFFFF0000u;
      }
    }
  };
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int e0 = (c * G + g) * VEC;
    if (c < nfull) {  // uniform
      if constexpr (VEC > 1) {
        load_vec(c, e0);
      } else {
        a[c] = bits_of<TIn>(wr[e0]);
      }
    } else {
      if (VEC > 1 && e0 + VEC <= k) {
        if constexpr (VEC > 1) load_vec(c, e0);
      } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) a[c * VEC + v] = (e0 + v < k) ? bits_of<TIn>(wr[e0 + v]) : 0u;
      }
    }
  }

  __shared__ uint32_t red_max[kWaves];
  __shared__ unsigned long long red_sum[kWaves];

  // max |w|: the signed maximum of the bit patterns is the largest
  // non-negative element (if any), the unsigned maximum the negative element
  // of largest magnitude (if any, else the same largest non-negative one).
  int32_t smax = 0;
  uint32_t umax = 0;
#pragma unroll
  for (int i = 0; i < CAP; ++i) {
    smax = max(smax, static_cast<int32_t>(a[i]));
    umax = max(umax, a[i]);
  }
  uint32_t amax = max(static_cast<uint32_t>(smax), umax & 0x7FFFFFFFu);
  amax = wave_max_u32(amax);
  if constexpr (R > 1) {
    if (lane == 0) red_max[wave] = amax;
    __syncthreads();
    amax = red_max[grp * R];
#pragma unroll
    for (int i = 1; i < R; ++i) amax = max(amax, red_max[grp * R + i]);
  }

  // E = floor(log2(max |w|)); every |w| < 2^(E+1), so every term < 2^49 and
  // a group of 16 sums to less than 2^53.  An all-zero row (amax == 0) sums
  // to zero and gets s = 0; the barrier below is outside every condition that
  // can differ between the rows of a workgroup.
  const int E = amax != 0u ? floor_log2_bits(amax) : 0;
  unsigned long long q = 0;
  if (amax != 0u) {
    const int sh = 48 - E;
#pragma unroll
    for (int g0 = 0; g0 < CAP; g0 += 16) {
      double acc = 0.0;
#pragma unroll
      for (int i = g0; i < (g0 + 16 < CAP ? g0 + 16 : CAP); ++i) acc += fixed_point_term(a[i], sh);
      q += u64_of(acc);
    }
  }
  q = wave_sum_u64(q);
  if constexpr (R > 1) {
    if (lane == 0) red_sum[wave] = q;
    __syncthreads();
    q = 0;
#pragma unroll
    for (int i = 0; i < R; ++i) q += red_sum[grp * R + i];
  }
  const float scale = amax != 0u ? scale_of(q, E, k) : 0.0f;
  if (g == 0 && valid) s[row] = scale;
  const float h = half_toward_zero(scale);

  // T = sign(w) where 2|w| > s, else 0.  An all-zero row has s = 0 and every
  // |w| = 0, so it also yields T = 0; elements past the row are zero and give
  // the zero fields that the packed format requires there.
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int e0 = (c * G + g) * VEC;
    if constexpr (VEC == 1) {
      const uint32_t code = code_of(a[c], h);
      if (pr != nullptr) {
        // Four consecutive weights sit in four neighbouring lanes (e0 % 4 is
        // g % 4): OR their fields together, the first of the four writes.
        uint32_t b = (code & 3u) << (2 * (e0 & 3));
        b |= __shfl_xor(b, 1, 64);
        b |= __shfl_xor(b, 2, 64);
        if ((e0 & 3) == 0 && e0 / 4 < nbytes) pr[e0 / 4] = static_cast<uint8_t>(b);
      }
      if (tr != nullptr && e0 < k) tr[e0] = static_cast<int8_t>(code);
    } else {
      uint32_t word[VEC / 4];
#pragma unroll
      for (int q = 0; q < VEC / 4; ++q)
        word[q] = gather4(code_of(a[c * VEC + 4 * q], h), code_of(a[c * VEC + 4 * q + 1], h),
                          code_of(a[c * VEC + 4 * q + 2], h), code_of(a[c * VEC + 4 * q + 3], h));
      auto store_vec = [&]() {
        if (pr != nullptr) {
#pragma unroll
          for (int q = 0; q < VEC / 4; ++q) pr[e0 / 4 + q] = static_cast<uint8_t>(pack4(word[q]));
        }
        if (tr != nullptr) {
          if constexpr (VEC == 4) {
            *reinterpret_cast<uint32_t*>(tr + e0) = word[0];
          } else {
            *reinterpret_cast<uint2*>(tr + e0) = make_uint2(word[0], word[1]);
          }
        }
      };
      if (c < nfull) {  // uniform
        store_vec();
      } else if (e0 + VEC <= k) {
        store_vec();
      } else {
        if (pr != nullptr) {
#pragma unroll
          for (int q = 0; q < VEC / 4; ++q)
            if (e0 / 4 + q < nbytes) pr[e0 / 4 + q] = static_cast<uint8_t>(pack4(word[q]));
        }
        if (tr != nullptr) {
#pragma unroll
          for (int v = 0; v < VEC; ++v)
            if (e0 + v < k) tr[e0 + v] = static_cast<int8_t>(word[v / 4] >> (8 * (v % 4)));
        }
      }
    }
  }
}

template <typename TIn, int VEC, int CAP, int R>
hipError_t launch_one(const TIn* w, int64_t n, int64_t k, int64_t ldw, int8_t* t, int64_t ldt,
                      float* s, uint8_t* p, int64_t ldp, hipStream_t stream) {
  constexpr int kRowsPerBlock = kWaves / R;
  const dim3 grid(static_cast<unsigned>((n + kRowsPerBlock - 1) / kRowsPerBlock)), block(kThreads);
  hipLaunchKernelGGL((quantize_rows<TIn, VEC, CAP, R>), grid, block, 0, stream, w, n,
                     static_cast<int>(k), ldw, t, ldt, s, p, ldp);
  return hipGetLastError();
}

// Elements per thread for a row of k over G threads in chunks of VEC.
inline int64_t per_thread(int64_t k, int g, int vec) {
  return (k + int64_t(g) * vec - 1) / (int64_t(g) * vec) * vec;
}

// The smallest listed capacity (a multiple of VEC) that holds `need`
// elements per thread; the list wastes at most a few elements for the row
// lengths in use.
template <typename TIn, int VEC, int R, int CAP, int... MORE>
hipError_t launch_caps(int64_t need, const TIn* w, int64_t n, int64_t k, int64_t ldw, int8_t* t,
                       int64_t ldt, float* s, uint8_t* p, int64_t ldp, hipStream_t stream) {
  if constexpr (CAP % VEC == 0) {
    if (need <= CAP) return launch_one<TIn, VEC, CAP, R>(w, n, k, ldw, t, ldt, s, p, ldp, stream);
  }
  if constexpr (sizeof...(MORE) > 0) {
    return launch_caps<TIn, VEC, R, MORE...>(need, w, n, k, ldw, t, ldt, s, p, ldp, stream);
  } else {
    return hipErrorInvalidValue;  // k > 32768 is rejected before this point
  }
}

// Waves per row: the fewest of 1, 2, 4 (at least kMinWavesPerRow) that keep
// a lane at 48 elements or fewer, else 4 (up to 128 per lane).
constexpr int kMinWavesPerRow = 1;

template <typename TIn, int VEC>
hipError_t launch_vec(const TIn* w, int64_t n, int64_t k, int64_t ldw, int8_t* t, int64_t ldt,
                      float* s, uint8_t* p, int64_t ldp, hipStream_t stream) {
  int64_t need = per_thread(k, 64, VEC);
  if (kMinWavesPerRow <= 1 && need <= 48)
    return launch_caps<TIn, VEC, 1, 4, 8, 12, 16, 20, 24, 28, 32, 40, 48>(
        need, w, n, k, ldw, t, ldt, s, p, ldp, stream);
  need = per_thread(k, 128, VEC);
  if (kMinWavesPerRow <= 2 && need <= 48)
    return launch_caps<TIn, VEC, 2, 4, 8, 12, 16, 20, 24, 28, 32, 40, 48>(
        need, w, n, k, ldw, t, ldt, s, p, ldp, stream);
  need = per_thread(k, 256, VEC);
  return launch_caps<TIn, VEC, 4, 4, 8, 12, 16, 20, 24, 28, 32, 40, 48, 64, 96, 128>(
      need, w, n, k, ldw, t, ldt, s, p, ldp, stream);
}

// Element-wise loads (unaligned rows): the workgroup owns the row.
template <typename TIn>
hipError_t launch_scalar(const TIn* w, int64_t n, int64_t k, int64_t ldw, int8_t* t, int64_t ldt,
                         float* s, uint8_t* p, int64_t ldp, hipStream_t stream) {
  return launch_caps<TIn, 1, 4, 8, 16, 32, 64, 128>(per_thread(k, 256, 1), w, n, k, ldw, t, ldt,
                                                    s, p, ldp, stream);
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

hipError_t launch_quantize(const void* w, bool w_is_bf16, int64_t n, int64_t k, int64_t ldw,
                           int8_t* t, int64_t ldt, float* s, uint8_t* p, int64_t ldp,
                           hipStream_t stream) {
  // Vector loads (and vector stores of the codes) where the rows allow them.
  const bool t_vec4 = t == nullptr || (aligned(t, 4) && ldt % 4 == 0);
  const bool t_vec8 = t == nullptr || (aligned(t, 8) && ldt % 8 == 0);
  if (!w_is_bf16) {
    const float* wf = static_cast<const float*>(w);
    if (aligned(w, 16) && ldw % 4 == 0 && t_vec4)
      return launch_vec<float, 4>(wf, n, k, ldw, t, ldt, s, p, ldp, stream);
    return launch_scalar<float>(wf, n, k, ldw, t, ldt, s, p, ldp, stream);
  }
  const uint16_t* wb = static_cast<const uint16_t*>(w);
  if (aligned(w, 16) && ldw % 8 == 0 && t_vec8)
    return launch_vec<uint16_t, 8>(wb, n, k, ldw, t, ldt, s, p, ldp, stream);
  return launch_scalar<uint16_t>(wb, n, k, ldw, t, ldt, s, p, ldp, stream);
}

}  // namespace tern
