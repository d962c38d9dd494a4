// Ternary linear layer for a handful of tokens (m <= 32):
// Y = bf16((X . T^T) (.) s), bf16 X, 2-bit packed T.
//
// "1.58-bit FLUX" (arXiv 2412.18653) stores the transformer's linear weights
// as 2-bit signed integers and keeps activations in 16 bits (section 1
// contributions, section 3.2, section 4 limitations).  With one or a few
// tokens per call the layer reads every packed weight once and does little
// arithmetic per byte, so this path is built around the weight stream: every
// weight byte is fetched exactly once, straight into registers, with as many
// fetches in flight per wave as its registers allow.
//
// Design:
//  * A workgroup owns 16 output channels (one MFMA A operand) and its four
//    waves split K: wave w takes the 256-wide K chunks w, w + 4, w + 8, ...
//    This gives N / 16 workgroups (288 for a 4608-wide layer), enough to keep
//    every CU fetching even for small layers.
//  * Lane (r, g) of a wave (r = lane % 16, g = lane / 16) fetches 16 bytes of
//    weight row r per chunk: codes 64 g .. 64 g + 63 of the chunk.  MFMA j of
//    the chunk (j = 0..7) uses codes 8 j .. 8 j + 7 of them, decoded in
//    registers to bf16 0 / +2 / -2 (the factor 2 is removed in the epilogue),
//    and the B operand is the matching 16-byte piece of X for token r (plus
//    16 per extra MFMA row block).  X is small and stays in L2.
//  * Loads use buffer resources: rows past n and tokens past m read as zero;
//    the part of a last chunk past k is read at an out-of-range offset, so it
//    is zero as well.
//  * The four per-wave partial sums are added through LDS; wave 0 applies the
//    fp32 channel scale and rounds once to bf16.
//  * A8 (int8 activations, the 8-bit-activation variant of the layer): the
//    weights come field-transposed, so one shift and one mask per register
//    give the int8 operand of v_mfma_i32_16x16x64_i8; MFMA d of a chunk
//    (d = 0..3) takes code word d of the lane's 16 bytes (codes 16 d .. 16 d
//    + 15 of its 64) and the matching 16 int8 values of X.  The partial sums
//    are exact int32 values and are added as integers; wave 0 converts the
//    total once and applies s[n] / 64 and the token's scale xs[m], the
//    formula of the tiled kernel, so both give the same bits.
#include <type_traits>

#include "gemm_common.h"
#include "internal.h"

namespace tern {
namespace {

constexpr int kSmallThreads = 256;
constexpr int kChunk = 256;           // K per chunk and wave
constexpr uint32_t kOutOfRange = 0x80000000u;

// R MFMA row blocks (m <= 16 R), B blocks of 16 output channels per
// workgroup (every wave covers all of them for its K chunks, so one X operand
// serves B MFMAs), DEPTH chunks in flight per wave.  With EPI the epilogue
// adds bias[n] (when bias is not null) and applies the tanh-form GELU to
// columns n >= act_from.
template <int R, int B, int DEPTH, bool EPI, bool A8 = false>
__global__ __launch_bounds__(kSmallThreads) void gemm_ternary_small(
    const uint8_t* __restrict__ x, int m, int k, int ldx, const float* __restrict__ xs,
    const uint8_t* __restrict__ p, int n, int ldp, const float* __restrict__ s,
    const float* __restrict__ bias, int act_from, uint16_t* __restrict__ y, int ldy,
    int y_vec_ok) {
  constexpr int kXElem = A8 ? 1 : 2;          // bytes per X element
  constexpr int kXPieces = A8 ? 4 : 8;        // 16-byte X pieces per chunk and lane
  __shared__ f32x4_t red[kSmallThreads / 64 - 1][B][R][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int n0 = blockIdx.x * (16 * B);
  const int rows = (n - n0) < 16 * B ? (n - n0) : 16 * B;

  const __amdgpu_buffer_rsrc_t prs = make_rsrc(
      p + static_cast<int64_t>(n0) * ldp, static_cast<uint32_t>((rows - 1) * ldp + k / 4));
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(
      x, static_cast<uint32_t>(((static_cast<int64_t>(m) - 1) * ldx + k) * kXElem));

  const int chunks = (k + kChunk - 1) / kChunk;
  const int mine = (chunks - wave + 3) / 4;  // chunks wave, wave + 4, ...

  // Per-lane byte offsets of chunk 0; chunk c adds c * kChunk codes.
  const uint32_t p_off = static_cast<uint32_t>(r16 * ldp + 16 * g);
  uint32_t x_off[R];
#pragma unroll
  for (int b = 0; b < R; ++b)
    x_off[b] = static_cast<uint32_t>(((16 * b + r16) * ldx + 64 * g) * kXElem);

  u32x4_t wq[DEPTH][B];
  u32x4_t xq[DEPTH][R][kXPieces];
  // Each chunk's loads are issued as one group, in chunk order (the fences
  // keep the scheduler from interleaving groups), so that waiting for the
  // oldest chunk never waits for a younger one.
  auto fence = []() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto fetch = [&](int slot, int c) {
    fence();
    // Codes kc .. kc + 63 of this lane lie past k exactly when kc >= k; then
    // the offsets get the out-of-range bit (arithmetic, so that the compiler
    // keeps one unconditional load per operand).
    const int kc = c * kChunk + 64 * g;
    const uint32_t oob = static_cast<uint32_t>(k - 1 - kc) & kOutOfRange;
#pragma unroll
    for (int bl = 0; bl < B; ++bl) {
      const uint32_t po =
          (p_off + static_cast<uint32_t>(bl * 16 * ldp + c * (kChunk / 4))) | oob;
      wq[slot][bl] =
          __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(prs, po, 0, 0));
    }
#pragma unroll
    for (int b = 0; b < R; ++b)
#pragma unroll
      for (int j = 0; j < kXPieces; ++j) {
        const uint32_t xo = (x_off[b] + static_cast<uint32_t>(c * kChunk * kXElem + 16 * j)) | oob;
        xq[slot][b][j] =
            __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xrs, xo, 0, 0));
      }
    fence();
  };

  // The channel scales of this lane's outputs, requested before the weight
  // stream so that they have arrived by the epilogue (a late request would
  // put a whole memory latency after the last MFMA).
  float sc[B][4];
#pragma unroll
  for (int bl = 0; bl < B; ++bl)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int nc = n0 + 16 * bl + 4 * g + e;
      sc[bl][e] = nc < n ? (s != nullptr ? s[nc] : 1.0f) * (A8 ? 0.015625f : 0.5f) : 0.0f;
    }
  float bsv[EPI ? B : 1][4];
  if constexpr (EPI) {
#pragma unroll
    for (int bl = 0; bl < B; ++bl)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int nc = n0 + 16 * bl + 4 * g + e;
        bsv[bl][e] = (bias != nullptr && nc < n) ? bias[nc] : 0.0f;
      }
  }

  f32x4_t acc[B][R];
#pragma unroll
  for (int bl = 0; bl < B; ++bl)
#pragma unroll
    for (int b = 0; b < R; ++b) acc[bl][b] = f32x4_t{};
  auto compute = [&](int slot) {
    if constexpr (A8) {
#pragma unroll
      for (int bl = 0; bl < B; ++bl)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          u32x4_t a;
#pragma unroll
          for (int r = 0; r < 4; ++r) a[r] = (wq[slot][bl][d] << (6 - 2 * r)) & 0xC0C0C0C0u;
#pragma unroll
          for (int b = 0; b < R; ++b) mfma_i8<false>(acc[bl][b], a, xq[slot][b][d]);
        }
      return;
    }
#pragma unroll
    for (int bl = 0; bl < B; ++bl)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        bf16x8_t lo, hi;
        decode16(wq[slot][bl][d], lo, hi);
#pragma unroll
        for (int b = 0; b < R; ++b) {
          mfma16<false>(acc[bl][b], lo, __builtin_bit_cast(bf16x8_t, xq[slot][b][2 * d]));
          mfma16<false>(acc[bl][b], hi, __builtin_bit_cast(bf16x8_t, xq[slot][b][2 * d + 1]));
        }
      }
  };

  // The wave's i-th chunk is global chunk wave + 4 i, fetched DEPTH chunks
  // ahead of its use into register slot i % DEPTH.  Fetches and MFMAs run
  // unconditionally in whole rounds of DEPTH chunks (chunks past the end read
  // as zero), so that the compiler's wait counts stay exact.
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) fetch(d, wave + 4 * d);
  for (int i0 = 0; i0 < mine; i0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      compute(d);
      fetch(d, wave + 4 * (i0 + d + DEPTH));
    }
  }

  // MFMA results may be read by other instructions only after up to 19 wait
  // states; the empty asm statements keep every read of acc after them.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int bl = 0; bl < B; ++bl)
#pragma unroll
    for (int b = 0; b < R; ++b) asm volatile("" : "+v"(acc[bl][b]));

  if (wave > 0) {
#pragma unroll
    for (int bl = 0; bl < B; ++bl)
#pragma unroll
      for (int b = 0; b < R; ++b) red[wave - 1][bl][b][lane] = acc[bl][b];
  }
  __syncthreads();
  if (wave != 0) return;

#pragma unroll
  for (int bl = 0; bl < B; ++bl) {
  const int nb = n0 + 16 * bl + 4 * g;  // output channels nb .. nb + 3 of this lane
#pragma unroll
  for (int b = 0; b < R; ++b) {
    f32x4_t v;
    if constexpr (A8) {
      i32x4_t vi = __builtin_bit_cast(i32x4_t, acc[bl][b]);
#pragma unroll
      for (int w = 0; w < kSmallThreads / 64 - 1; ++w)
        vi += __builtin_bit_cast(i32x4_t, red[w][bl][b][lane]);
      v = __builtin_convertvector(vi, f32x4_t);
    } else {
      v = acc[bl][b];
#pragma unroll
      for (int w = 0; w < kSmallThreads / 64 - 1; ++w) v += red[w][bl][b][lane];
    }
    const int token = 16 * b + r16;
    if (token >= m) continue;
    float xsm = 1.0f;
    if constexpr (A8) xsm = xs[token];
    __bf16 o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float z = v[e] * sc[bl][e];
      if constexpr (A8) z *= xsm;
      if constexpr (EPI) {
        z += bsv[bl][e];
        if (nb + e >= act_from) z = gelu_tanh_f32(z);
      }
      o[e] = static_cast<__bf16>(z);
    }
    uint16_t* yr = y + static_cast<int64_t>(token) * ldy + nb;
    if (y_vec_ok && nb + 4 <= n) {
      u32x2_t q;
      q[0] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, o[0])) |
             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, o[1])) << 16);
      q[1] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, o[2])) |
             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, o[3])) << 16);
      *reinterpret_cast<u32x2_t*>(yr) = q;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (nb + e < n) yr[e] = __builtin_bit_cast(uint16_t, o[e]);
    }
  }
  }
}

template <int R, int B, int DEPTH, bool EPI, bool A8>
hipError_t launch_small(const void* x, int64_t m, int64_t k, int64_t ldx, const float* xs,
                        const uint8_t* p, int64_t n, int64_t ldp, const float* s,
                        const float* bias, int act_from, uint16_t* y, int64_t ldy,
                        hipStream_t stream) {
  const int64_t blocks = (n + 16 * B - 1) / (16 * B);
  const int y_vec_ok = ((reinterpret_cast<uintptr_t>(y) & 7) == 0) && (ldy % 4 == 0);
  hipLaunchKernelGGL((gemm_ternary_small<R, B, DEPTH, EPI, A8>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kSmallThreads), 0, stream, static_cast<const uint8_t*>(x),
                     static_cast<int>(m), static_cast<int>(k), static_cast<int>(ldx), xs, p,
                     static_cast<int>(n), static_cast<int>(ldp), s, bias, act_from, y,
                     static_cast<int>(ldy), y_vec_ok);
  return hipGetLastError();
}


template <bool EPI, bool A8 = false>
hipError_t launch_small_any(const void* x, int64_t m, int64_t k, int64_t ldx, const float* xs,
                            const uint8_t* p, int64_t n, int64_t ldp, const float* s,
                            const float* bias, int act_from, uint16_t* y, int64_t ldy,
                            hipStream_t stream) {
  // Channel blocks per workgroup.  The weight stream is latency-bound: every
  // CU keeps a fixed number of bytes in flight per workgroup, and a CU that
  // holds two workgroups finishes them well after the CUs that hold one.  So
  // B is chosen to minimize the blocks of the busiest CU, B * ceil(ceil(nb /
  // B) / 256) for nb blocks of 16 channels, the larger B on ties (each X
  // operand then feeds B MFMAs).  E.g. N = 21504: B = 6, 224 workgroups,
  // instead of 336 with B = 4.
  const int64_t nb = (n + 15) / 16;
  int best = 1;
  int64_t best_cost = -1;
  for (int b : {6, 3, 2, 1}) {
    const int64_t wgs = (nb + b - 1) / b;
    const int64_t cost = b * ((wgs + 255) / 256);
    if (best_cost < 0 || cost < best_cost) {
      best = b;
      best_cost = cost;
    }
  }
#define TERN_SMALL(R, DEPTH6, DEPTH3, DEPTH2, DEPTH1)                                           \
  switch (best) {                                                                               \
    case 6:                                                                                     \
      return launch_small<R, 6, DEPTH6, EPI, A8>(x, m, k, ldx, xs, p, n, ldp, s, bias, act_from, \
                                                 y, ldy, stream);                                 \
    case 3:                                                                                     \
      return launch_small<R, 3, DEPTH3, EPI, A8>(x, m, k, ldx, xs, p, n, ldp, s, bias, act_from, \
                                                 y, ldy, stream);                                 \
    case 2:                                                                                     \
      return launch_small<R, 2, DEPTH2, EPI, A8>(x, m, k, ldx, xs, p, n, ldp, s, bias, act_from, \
                                                 y, ldy, stream);                                 \
    default:                                                                                    \
      return launch_small<R, 1, DEPTH1, EPI, A8>(x, m, k, ldx, xs, p, n, ldp, s, bias, act_from, \
                                                 y, ldy, stream);                                 \
  }
  if (m <= 16) TERN_SMALL(1, 3, 3, 4, 4)
  TERN_SMALL(2, 2, 2, 2, 2)
#undef TERN_SMALL
}

}  // namespace

hipError_t launch_gemm_small(const uint16_t* x, int64_t m, int64_t k, int64_t ldx,
                             const uint8_t* p, int64_t n, int64_t ldp, const float* s,
                             const float* bias, int64_t act_from, uint16_t* y, int64_t ldy,
                             hipStream_t stream) {
  if (bias != nullptr || act_from < n)
    return launch_small_any<true>(x, m, k, ldx, nullptr, p, n, ldp, s, bias,
                                  static_cast<int>(act_from), y, ldy, stream);
  return launch_small_any<false>(x, m, k, ldx, nullptr, p, n, ldp, s, nullptr,
                                 static_cast<int>(act_from), y, ldy, stream);
}

hipError_t launch_gemm_small_a8(const int8_t* q, int64_t m, int64_t k, int64_t ldq,
                                const float* xs, const uint8_t* p8, int64_t n, int64_t ldp8,
                                const float* s, const float* bias, int64_t act_from, uint16_t* y,
                                int64_t ldy, hipStream_t stream) {
  if (bias != nullptr || act_from < n)
    return launch_small_any<true, true>(q, m, k, ldq, xs, p8, n, ldp8, s, bias,
                                        static_cast<int>(act_from), y, ldy, stream);
  return launch_small_any<false, true>(q, m, k, ldq, xs, p8, n, ldp8, s, nullptr,
                                       static_cast<int>(act_from), y, ldy, stream);
}

}  // namespace tern
