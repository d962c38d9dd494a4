// The 8-bit-activation (W1.58-A8) inputs of the ternary layer: per-token
// int8 activations and the field-transposed weight codes.
//
// "1.58-bit FLUX" (section 4, limitations) names the absence of activation
// quantization as the reason its latency barely improved; the pages define no
// activation quantizer.  The plainest one, absmax per token (as in the BitNet
// b1.58 family the paper builds on, section 1), is used here:
//   g_m = max(max_k |x[m][k]|, 1e-5),
//   q[m][k] = rint(fp32(x[m][k] * fp32(127 / g_m))),  xs[m] = fp32(g_m / 127),
// with every quotient correctly rounded to fp32 and ties to even.  The floor
// keeps 127 / g finite (it overflows fp32 below about 3.7e-37); a row of
// zeros gives q = 0.  |q| <= 127 follows from |x| <= g.
//
// quantize_act: HBM-bound (2 bytes read, 1 written per element).  One wave
// per token.  Rows of up to 16384 elements (with 16-byte aligned rows) are
// read once into registers, 8 elements per lane per 1 KiB chunk of the row;
// the absolute maximum comes from a butterfly over the wave and the codes
// are written from the registers.  Other rows take two passes, the second
// re-reading the row (from HBM at large sizes: with every CU streaming rows
// the cache does not keep a row between the passes).
//
// pack_a8: the int8 MFMA operand of 16 codes is four registers of four
// bytes in ascending k.  With the 2-bit fields of each 32-bit code word
// transposed as a 4 x 4 matrix (field 4 i + j holds code 4 j + i), one shift
// and one mask, (w << (6 - 2 r)) & 0xC0C0C0C0, give register r directly:
// byte b holds code 4 r + b in bits 6..7, the int8 value 0 / +64 / -64.  The
// transposition is two delta swaps per word (it is its own inverse).
#include "internal.h"

namespace tern {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int64_t kMaxBlocks = 256 * 64;

__device__ inline float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Four int8 codes of four fp32 values already scaled to [-127, 127]: round
// to nearest even, convert, keep the low bytes (byte e from value e).
__device__ inline uint32_t pack_codes4(float a, float b, float c, float d) {
  const uint32_t qa = static_cast<uint32_t>(static_cast<int>(__builtin_rintf(a))) & 0xFFu;
  const uint32_t qb = static_cast<uint32_t>(static_cast<int>(__builtin_rintf(b))) & 0xFFu;
  const uint32_t qc = static_cast<uint32_t>(static_cast<int>(__builtin_rintf(c))) & 0xFFu;
  const uint32_t qd = static_cast<uint32_t>(static_cast<int>(__builtin_rintf(d))) & 0xFFu;
  return qa | (qb << 8) | (qc << 16) | (qd << 24);
}

// VEC: x rows start 16-byte aligned, q rows 8-byte aligned and k % 8 == 0;
// each lane then handles 8 consecutive elements per access.  Otherwise one
// element per lane per access.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void quantize_act_kernel(const uint16_t* __restrict__ x,
                                                                int64_t m, int64_t k, int64_t ldx,
                                                                int8_t* __restrict__ q, int64_t ldq,
                                                                float* __restrict__ xs) {
  const int lane = threadIdx.x & 63;
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6); row < m;
       row += static_cast<int64_t>(gridDim.x) * kWaves) {
    const uint16_t* xr = x + row * ldx;
    int8_t* qr = q + row * ldq;
    // Pass 1: absolute maximum (bf16 values are exact in fp32; the bit
    // pattern of |v| orders like its value).
    uint32_t amax = 0;
    if constexpr (VEC) {
      for (int64_t c = 8 * lane; c < k; c += 512) {
        const uint4 v = *reinterpret_cast<const uint4*>(xr + c);
        const uint32_t a0 = (v.x & 0x7FFFu) > ((v.x >> 16) & 0x7FFFu) ? (v.x & 0x7FFFu) : ((v.x >> 16) & 0x7FFFu);
        const uint32_t a1 = (v.y & 0x7FFFu) > ((v.y >> 16) & 0x7FFFu) ? (v.y & 0x7FFFu) : ((v.y >> 16) & 0x7FFFu);
        const uint32_t a2 = (v.z & 0x7FFFu) > ((v.z >> 16) & 0x7FFFu) ? (v.z & 0x7FFFu) : ((v.z >> 16) & 0x7FFFu);
        const uint32_t a3 = (v.w & 0x7FFFu) > ((v.w >> 16) & 0x7FFFu) ? (v.w & 0x7FFFu) : ((v.w >> 16) & 0x7FFFu);
        const uint32_t b01 = a0 > a1 ? a0 : a1;
        const uint32_t b23 = a2 > a3 ? a2 : a3;
        const uint32_t b = b01 > b23 ? b01 : b23;
        amax = amax > b ? amax : b;
      }
    } else {
      for (int64_t c = lane; c < k; c += 64) {
        const uint32_t a = xr[c] & 0x7FFFu;
        amax = amax > a ? amax : a;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), off));
      amax = amax > o ? amax : o;
    }
    const float g = fmaxf(__uint_as_float(amax << 16), 1e-5f);
    // Correctly rounded fp32 quotients: the double quotient of two floats
    // rounded to float is the correctly rounded float quotient (53 >= 2 * 24 + 2).
    const float inv = static_cast<float>(127.0 / static_cast<double>(g));
    if (lane == 0) xs[row] = static_cast<float>(static_cast<double>(g) / 127.0);
    // Pass 2: the codes.
    if constexpr (VEC) {
      for (int64_t c = 8 * lane; c < k; c += 512) {
        const uint4 v = *reinterpret_cast<const uint4*>(xr + c);
        uint2 o;
        o.x = pack_codes4(bf16_lo(v.x) * inv, bf16_hi(v.x) * inv, bf16_lo(v.y) * inv,
                          bf16_hi(v.y) * inv);
        o.y = pack_codes4(bf16_lo(v.z) * inv, bf16_hi(v.z) * inv, bf16_lo(v.w) * inv,
                          bf16_hi(v.w) * inv);
        *reinterpret_cast<uint2*>(qr + c) = o;
      }
    } else {
      for (int64_t c = lane; c < k; c += 64)
        qr[c] = static_cast<int8_t>(static_cast<int>(__builtin_rintf(bf16_lo(xr[c]) * inv)));
    }
  }
}

// The larger of the absolute values of the two bf16 halves of v, as a
// 15-bit pattern (for finite values the pattern orders like the value).
__device__ inline uint32_t abs2(uint32_t v) {
  const uint32_t a = v & 0x7FFFu, b = (v >> 16) & 0x7FFFu;
  return a > b ? a : b;
}

__device__ inline uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off));
    v = v > o ? v : o;
  }
  return v;
}

// One pass: rows of at most 512 * CAP elements, x rows 16-byte aligned, q
// rows 8-byte aligned, k % 8 == 0.  Chunk c of a row is elements 512 c ..
// 512 c + 511; lane l holds elements 512 c + 8 l .. 512 c + 8 l + 7.
template <int CAP>
__global__ __launch_bounds__(kThreads) void quantize_act_regs_kernel(
    const uint16_t* __restrict__ x, int64_t m, int k, int64_t ldx, int8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ xs) {
  const int lane = threadIdx.x & 63;
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6); row < m;
       row += static_cast<int64_t>(gridDim.x) * kWaves) {
    const uint16_t* xr = x + row * ldx;
    int8_t* qr = q + row * ldq;
    uint4 v[CAP];
#pragma unroll
    for (int c = 0; c < CAP; ++c) {
      const int e = 512 * c + 8 * lane;
      v[c] = e < k ? *reinterpret_cast<const uint4*>(xr + e) : uint4{0u, 0u, 0u, 0u};
    }
    uint32_t amax = 0;
#pragma unroll
    for (int c = 0; c < CAP; ++c) {
      const uint32_t a = abs2(v[c].x) > abs2(v[c].y) ? abs2(v[c].x) : abs2(v[c].y);
      const uint32_t b = abs2(v[c].z) > abs2(v[c].w) ? abs2(v[c].z) : abs2(v[c].w);
      const uint32_t ab = a > b ? a : b;
      amax = amax > ab ? amax : ab;
    }
    amax = wave_max(amax);
    const float g = fmaxf(__uint_as_float(amax << 16), 1e-5f);
    const float inv = static_cast<float>(127.0 / static_cast<double>(g));
    if (lane == 0) xs[row] = static_cast<float>(static_cast<double>(g) / 127.0);
#pragma unroll
    for (int c = 0; c < CAP; ++c) {
      const int e = 512 * c + 8 * lane;
      if (e < k) {
        uint2 o;
        o.x = pack_codes4(bf16_lo(v[c].x) * inv, bf16_hi(v[c].x) * inv, bf16_lo(v[c].y) * inv,
                          bf16_hi(v[c].y) * inv);
        o.y = pack_codes4(bf16_lo(v[c].z) * inv, bf16_hi(v[c].z) * inv, bf16_lo(v[c].w) * inv,
                          bf16_hi(v[c].w) * inv);
        *reinterpret_cast<uint2*>(qr + e) = o;
      }
    }
  }
}

__device__ inline uint32_t transpose_fields(uint32_t w) {
  uint32_t t = ((w >> 12) ^ w) & 0x0000F0F0u;  // off-diagonal 2 x 2 blocks of fields
  w ^= t ^ (t << 12);
  t = ((w >> 6) ^ w) & 0x00CC00CCu;            // off-diagonal fields within each block
  return w ^ t ^ (t << 6);
}

// One 16-byte group (4 words) per thread when VEC (pointers 16-byte aligned,
// pitches multiples of 16, k % 64 == 0), else one word.
template <bool VEC, typename IDX>
__global__ __launch_bounds__(kThreads) void pack_a8_kernel(const uint8_t* __restrict__ p,
                                                           IDX n, IDX words, IDX ldp,
                                                           uint8_t* __restrict__ p8, IDX ldp8) {
  constexpr IDX kPer = VEC ? 4 : 1;
  const IDX per_row = words / kPer;
  const IDX total = n * per_row;
  for (IDX idx = static_cast<IDX>(blockIdx.x) * kThreads + threadIdx.x; idx < total;
       idx += static_cast<IDX>(gridDim.x) * kThreads) {
    const IDX row = idx / per_row;
    const IDX w = (idx - row * per_row) * kPer;
    if constexpr (VEC) {
      uint4 v = *reinterpret_cast<const uint4*>(p + row * ldp + 4 * w);
      v.x = transpose_fields(v.x);
      v.y = transpose_fields(v.y);
      v.z = transpose_fields(v.z);
      v.w = transpose_fields(v.w);
      *reinterpret_cast<uint4*>(p8 + row * ldp8 + 4 * w) = v;
    } else {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(p + row * ldp + 4 * w);
      *reinterpret_cast<uint32_t*>(p8 + row * ldp8 + 4 * w) = transpose_fields(v);
    }
  }
}

}  // namespace

hipError_t launch_quantize_act(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, int8_t* q,
                               int64_t ldq, float* xs, hipStream_t stream) {
  const bool vec = reinterpret_cast<uintptr_t>(x) % 16 == 0 && ldx % 8 == 0 && k % 8 == 0 &&
                   reinterpret_cast<uintptr_t>(q) % 8 == 0 && ldq % 8 == 0;
  int64_t blocks = (m + kWaves - 1) / kWaves;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (vec && k <= 16384) {
    const int ki = static_cast<int>(k);
    if (k <= 1024)
      hipLaunchKernelGGL(quantize_act_regs_kernel<2>, grid, dim3(kThreads), 0, stream, x, m, ki,
                         ldx, q, ldq, xs);
    else if (k <= 2048)
      hipLaunchKernelGGL(quantize_act_regs_kernel<4>, grid, dim3(kThreads), 0, stream, x, m, ki,
                         ldx, q, ldq, xs);
    else if (k <= 4096)
      hipLaunchKernelGGL(quantize_act_regs_kernel<8>, grid, dim3(kThreads), 0, stream, x, m, ki,
                         ldx, q, ldq, xs);
    else if (k <= 8192)
      hipLaunchKernelGGL(quantize_act_regs_kernel<16>, grid, dim3(kThreads), 0, stream, x, m, ki,
                         ldx, q, ldq, xs);
    else
      hipLaunchKernelGGL(quantize_act_regs_kernel<32>, grid, dim3(kThreads), 0, stream, x, m, ki,
                         ldx, q, ldq, xs);
    return hipGetLastError();
  }
  if (vec)
    hipLaunchKernelGGL(quantize_act_kernel<true>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, x, m, k, ldx, q, ldq, xs);
  else
    hipLaunchKernelGGL(quantize_act_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, x, m, k, ldx, q, ldq, xs);
  return hipGetLastError();
}

hipError_t launch_pack_a8(const uint8_t* p, int64_t n, int64_t k, int64_t ldp, uint8_t* p8,
                          int64_t ldp8, hipStream_t stream) {
  const int64_t words = k / 16;
  const bool vec = reinterpret_cast<uintptr_t>(p) % 16 == 0 && ldp % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(p8) % 16 == 0 && ldp8 % 16 == 0 && words % 4 == 0;
  const int64_t per = vec ? 4 : 1;
  const int64_t total = n * (words / per);
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  if (blocks < 1) blocks = 1;
  // 32-bit indexing when every index (and every byte offset) fits.
  const bool small = n * ldp < (int64_t(1) << 31) && n * ldp8 < (int64_t(1) << 31) &&
                     total + blocks * kThreads < (int64_t(1) << 31);
  const dim3 grid(static_cast<unsigned>(blocks));
  if (vec && small)
    hipLaunchKernelGGL((pack_a8_kernel<true, uint32_t>), grid, dim3(kThreads), 0, stream, p,
                       static_cast<uint32_t>(n), static_cast<uint32_t>(words),
                       static_cast<uint32_t>(ldp), p8, static_cast<uint32_t>(ldp8));
  else if (vec)
    hipLaunchKernelGGL((pack_a8_kernel<true, int64_t>), grid, dim3(kThreads), 0, stream, p, n,
                       words, ldp, p8, ldp8);
  else if (small)
    hipLaunchKernelGGL((pack_a8_kernel<false, uint32_t>), grid, dim3(kThreads), 0, stream, p,
                       static_cast<uint32_t>(n), static_cast<uint32_t>(words),
                       static_cast<uint32_t>(ldp), p8, static_cast<uint32_t>(ldp8));
  else
    hipLaunchKernelGGL((pack_a8_kernel<false, int64_t>), grid, dim3(kThreads), 0, stream, p, n,
                       words, ldp, p8, ldp8);
  return hipGetLastError();
}

}  // namespace tern
