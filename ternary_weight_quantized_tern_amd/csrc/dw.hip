// Gradient of the latent full-precision weights of the ternary layer:
//   dW[n][k] = (accumulate ? dW[n][k] : 0) + sum_m dY[m][n] * X[m][k]
// bf16 dY and X, fp32 dW.
//
// "TerDiT: Ternary Diffusion Models with Transformers" (abstract) trains the
// ternary weights of a DiT in the loop (quantization-aware training); the
// pages give no formula.  The layer is Y = X . (s (.) T)^T, and the reading
// used is the straight-through estimator that passes the gradient of the
// quantized weight s_n T_nk unchanged to the latent weight w_nk, so the
// latent weights receive dY^T . X: a dense bf16 contraction over the tokens,
// run on the bf16 matrix cores with fp32 accumulation.
//
// Design:
//  * The MFMA computes D = A . B with A = X^T (rows = input features k) and
//    B = dY (columns = output channels n), so that every lane ends up with
//    four consecutive k of one channel n: D[k][n] = dW[n][k], written as one
//    16-byte run of fp32 per MFMA tile.
//  * Both operands are token-major in memory (a row of X or dY is one token),
//    and the contraction runs over tokens.  A stage of 32 tokens of the X
//    columns of the tile and of the dY columns of the tile is copied as it is
//    into LDS with buffer loads in the LDS-DMA form, and the MFMA operands
//    are read with ds_read_b64_tr_b16, the gfx950 LDS read that transposes
//    16-bit elements within each group of 16 lanes: source lane 4 j + b of a
//    group reads 4 consecutive columns 4 b .. 4 b + 3 of token row j, and
//    lane i of the group receives column i of token rows 0..3 (measured lane
//    layout: destination lane i, element j <- source lane 4 j + i / 4,
//    element i % 4).  Two such reads (token rows 8 g .. 8 g + 3 and
//    8 g + 4 .. 8 g + 7) give lane (g, i) the 8 contraction values of column
//    i that v_mfma_f32_16x16x32_bf16 takes from it.
//  * The 16-byte chunks of each LDS row are XOR-swizzled by the row: chunk c
//    of token row r is stored in slot c ^ f(r), f(r) = 2 (r % 4) + 8 ((r / 8)
//    % 2); the swizzle is applied on the global side of the DMA.  A
//    transposed read of a group touches 4 token rows of one 32-byte column
//    window, which the swizzle spreads over 4 distinct 32-byte bank groups.
//  * A ring of four stages: three in flight while one is read, one barrier
//    per stage.  Tokens past m read as zero (buffer range check), and so do
//    the stages past the last one; columns past k or n hold values that only
//    reach outputs that are not stored.
//  * Tile 256 (k) x 256 (n) with four waves of 128 x 128 (8 x 8 MFMA tiles,
//    256 accumulator registers) where there are at least 256 such tiles,
//    else 128 x 128 with four waves of 64 x 64.
#include "gemm_common.h"
#include "internal.h"

namespace tern {
namespace {

constexpr int kDwThreads = 256;
constexpr int kSm = 32;    // tokens per stage
constexpr int kDwRing = 4; // stages in the ring

template <int N>
__device__ inline void dw_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that orders the LDS accesses for the compiler without the
// memory fence of __syncthreads() (which would also wait for every DMA in
// flight); DMA visibility comes from each wave's vmcnt wait before it.
__device__ inline void dw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ inline uint32_t dw_swz(uint32_t r) { return ((r & 3u) << 1) | (((r >> 3) & 1u) << 3); }

typedef __attribute__((ext_vector_type(4))) short i16x4_t;

template <int TK, int TN>
struct DwCfg {
  static constexpr int kWK = TK / 2;                 // wave tile (2 x 2 waves): k
  static constexpr int kWN = TN / 2;                 // ... n
  static constexpr int kTI = kWK / 16;               // MFMA tiles per wave along k
  static constexpr int kTJ = kWN / 16;               // ... along n
  static constexpr int kXBytes = kSm * TK * 2;       // X part of a stage
  static constexpr int kYBytes = kSm * TN * 2;       // dY part
  static constexpr int kStage = kXBytes + kYBytes;
  static constexpr int kXInstr = kXBytes / 1024;     // 1 KiB DMA instructions: X
  static constexpr int kYInstr = kYBytes / 1024;     // ... dY
  static constexpr int kInstr = kXInstr + kYInstr;
  static constexpr int kLoads = kInstr / 4;          // per wave and stage
  static_assert(TK >= 128 && TN >= 128 && TK % 128 == 0 && TN % 128 == 0, "tile");
  static_assert(kInstr % 4 == 0, "every wave issues the same number of loads");
};

template <int TK, int TN>
__global__ __launch_bounds__(kDwThreads) void gemm_dw_mfma(
    const uint16_t* __restrict__ dy, int m, int n, int lddy, const uint16_t* __restrict__ x, int k,
    int ldx, float* __restrict__ dw, int lddw, int accumulate, int tiles_k, int vec_ok) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = DwCfg<TK, TN>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[C::kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;   // contraction group of the MFMA operands
  const int sl = lane & 15;  // lane within its group

  // Tile of this workgroup.  Workgroups are dealt to the 8 XCDs round-robin;
  // renumbering gives each XCD a contiguous range of tiles, which walk k
  // fastest, so concurrent workgroups of an XCD share dY columns in its L2.
  const int grid = gridDim.x;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, per = grid >> 3, rem = grid & 7;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + (bid >> 3);
  const int k0 = (logical % tiles_k) * TK;
  const int n0 = (logical / tiles_k) * TN;
  const int wk0 = (wave & 1) * C::kWK;   // wave's offset in the tile: k
  const int wn0 = (wave >> 1) * C::kWN;  // ... n

  // DMA plan: load q of this wave is instruction gi = wave + 4 q of the
  // stage: X rows (tokens) 512 / TK per instruction, then dY rows.  Lane l
  // fills LDS bytes [1024 gi + 16 l, +16): token row r, slot p, which holds
  // the row's logical chunk p ^ f(r).
  uint32_t dma_voff[C::kLoads];
  uint32_t dma_lds[C::kLoads];
  bool dma_is_x[C::kLoads];
#pragma unroll
  for (int q = 0; q < C::kLoads; ++q) {
    const int gi = wave + 4 * q;
    dma_is_x[q] = gi < C::kXInstr;
    if (dma_is_x[q]) {
      constexpr int kCpr = TK / 8;  // 16-byte chunks per X row
      const uint32_t r = static_cast<uint32_t>(gi * (1024 / (2 * TK)) + lane / kCpr);
      const uint32_t c = static_cast<uint32_t>(lane % kCpr) ^ dw_swz(r);
      dma_voff[q] = r * static_cast<uint32_t>(ldx) * 2u + 16u * c;
      dma_lds[q] = 1024u * gi;
    } else {
      constexpr int kCpr = TN / 8;
      const int gy = gi - C::kXInstr;
      const uint32_t r = static_cast<uint32_t>(gy * (1024 / (2 * TN)) + lane / kCpr);
      const uint32_t c = static_cast<uint32_t>(lane % kCpr) ^ dw_swz(r);
      dma_voff[q] = r * static_cast<uint32_t>(lddy) * 2u + 16u * c;
      dma_lds[q] = C::kXBytes + 1024u * gy;
    }
  }

  // Buffer resources of stage st: rebased at the stage's first token and the
  // tile's first column; tokens past m fall outside num_records.  The range
  // check drops every 4-byte word that is not wholly inside it, so the last
  // row's range is rounded up to whole 16-byte chunks (an odd width would
  // otherwise lose its last element there); the caller's matrix extends that
  // far (rows are padded to a multiple of 8 elements).
  const int stages = (m + kSm - 1) / kSm;
  auto x_rsrc = [&](int st) {
    const int t0 = st * kSm;
    const uint32_t rec = t0 < m ? static_cast<uint32_t>((static_cast<int64_t>(m - t0 - 1) * ldx +
                                                         ((k - k0 + 7) & ~7)) * 2)
                                : 0u;
    return make_rsrc(x + static_cast<int64_t>(t0 < m ? t0 : 0) * ldx + k0, rec);
  };
  auto y_rsrc = [&](int st) {
    const int t0 = st * kSm;
    const uint32_t rec = t0 < m ? static_cast<uint32_t>((static_cast<int64_t>(m - t0 - 1) * lddy +
                                                         ((n - n0 + 7) & ~7)) * 2)
                                : 0u;
    return make_rsrc(dy + static_cast<int64_t>(t0 < m ? t0 : 0) * lddy + n0, rec);
  };
#define TERN_DW_ISSUE(BUF, ST)                                                                 \
  {                                                                                            \
    const __amdgpu_buffer_rsrc_t xr_ = x_rsrc(ST);                                             \
    const __amdgpu_buffer_rsrc_t yr_ = y_rsrc(ST);                                             \
    _Pragma("unroll") for (int q = 0; q < C::kLoads; ++q)                                      \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(dma_is_x[q] ? xr_ : yr_,                      \
                                                 (lds_void_t*)(&BUF[dma_lds[q]]), 16,          \
                                                 dma_voff[q], 0, 0, 0);                        \
  }

  // Transposed operand reads.  Lane (g, sl) reads token row 8 g + sl / 4 (and
  // 4 rows further for the second half of its 8 values), 4 columns starting
  // at 4 (sl % 4) of the 16-column block of its MFMA tile.
  const uint32_t r0 = static_cast<uint32_t>(8 * g + (sl >> 2));
  const uint32_t f0 = dw_swz(r0);
  const uint32_t half = static_cast<uint32_t>((sl >> 1) & 1);  // chunk within the 32-byte window
  const uint32_t sub = static_cast<uint32_t>((sl & 1) * 8);    // 8-byte half of the chunk
  uint32_t offa[C::kTI], offb[C::kTJ];
#pragma unroll
  for (int ti = 0; ti < C::kTI; ++ti) {
    const uint32_t c = (static_cast<uint32_t>((wk0 + 16 * ti) / 8) ^ f0) | half;
    offa[ti] = r0 * (2 * TK) + 16 * c + sub;
  }
#pragma unroll
  for (int tj = 0; tj < C::kTJ; ++tj) {
    const uint32_t c = (static_cast<uint32_t>((wn0 + 16 * tj) / 8) ^ f0) | half;
    offb[tj] = C::kXBytes + r0 * (2 * TN) + 16 * c + sub;
  }
  constexpr uint32_t kXRow4 = 4 * 2 * TK;  // 4 token rows further
  constexpr uint32_t kYRow4 = 4 * 2 * TN;

  f32x4_t acc[C::kTI][C::kTJ];
#pragma unroll
  for (int ti = 0; ti < C::kTI; ++ti)
#pragma unroll
    for (int tj = 0; tj < C::kTJ; ++tj) acc[ti][tj] = f32x4_t{};

  auto tr = [](const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(p));
  };
  auto operand = [](i16x4_t lo, i16x4_t hi) {
    u32x4_t v;
    const u32x2_t a = __builtin_bit_cast(u32x2_t, lo), b = __builtin_bit_cast(u32x2_t, hi);
    v[0] = a[0];
    v[1] = a[1];
    v[2] = b[0];
    v[3] = b[1];
    return v;
  };
  // The B operands of every n tile, then the A operand of k tile ti + 1 read
  // while the MFMAs of k tile ti run (two A registers sets, so that an LDS
  // read is always in flight behind the matrix cores).
#define TERN_DW_COMPUTE(BUF)                                                                     \
  {                                                                                              \
    u32x4_t bq[C::kTJ];                                                                          \
    u32x4_t aq[2];                                                                               \
    _Pragma("unroll") for (int tj = 0; tj < C::kTJ; ++tj) bq[tj] =                               \
        operand(tr(&BUF[offb[tj]]), tr(&BUF[offb[tj] + kYRow4]));                                \
    aq[0] = operand(tr(&BUF[offa[0]]), tr(&BUF[offa[0] + kXRow4]));                              \
    _Pragma("unroll") for (int ti = 0; ti < C::kTI; ++ti) {                                      \
      if (ti + 1 < C::kTI)                                                                       \
        aq[(ti + 1) & 1] = operand(tr(&BUF[offa[ti + 1]]), tr(&BUF[offa[ti + 1] + kXRow4]));     \
      _Pragma("unroll") for (int tj = 0; tj < C::kTJ; ++tj)                                      \
          mfma16<false, false>(acc[ti][tj], __builtin_bit_cast(bf16x8_t, aq[ti & 1]),             \
                              __builtin_bit_cast(bf16x8_t, bq[tj]));                             \
    }                                                                                            \
  }
  // One stage: wait until this wave's DMAs of the stage have landed (two
  // younger stages may still be in flight), meet at the barrier (every wave's
  // DMAs of the stage have landed and every wave is done with the previous
  // stage, whose buffer the next request refills), request the stage three
  // ahead, read and multiply.
#define TERN_DW_STEP(CUR, NXT, ST)               \
  dw_wait_vmcnt<2 * C::kLoads>();               \
  dw_barrier();                                 \
  TERN_DW_ISSUE(NXT, (ST) + kDwRing - 1)        \
  TERN_DW_COMPUTE(CUR)

  TERN_DW_ISSUE(lds0, 0)
  TERN_DW_ISSUE(lds1, 1)
  TERN_DW_ISSUE(lds2, 2)
  for (int st = 0; st < stages; st += kDwRing) {
    TERN_DW_STEP(lds0, lds3, st)
    TERN_DW_STEP(lds1, lds0, st + 1)
    TERN_DW_STEP(lds2, lds1, st + 2)
    TERN_DW_STEP(lds3, lds2, st + 3)
    // The loop's exit and back edge are joins where the compiler may move
    // accumulators between registers; 24 wait states after the last MFMA
    // make every result readable there.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  }
  dw_wait_vmcnt<0>();  // no DMA may outlive the workgroup's LDS
#undef TERN_DW_STEP
#undef TERN_DW_COMPUTE
#undef TERN_DW_ISSUE

  // MFMA results may be read by other instructions only after up to 19 wait
  // states; the empty asm statements keep every read of acc after them.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int ti = 0; ti < C::kTI; ++ti)
#pragma unroll
    for (int tj = 0; tj < C::kTJ; ++tj) asm volatile("" : "+a"(acc[ti][tj]));

  // Lane (g, sl) of MFMA tile (ti, tj) holds D[kk + e][nn], e = 0..3:
  // dW[nn][kk .. kk + 3] with nn = n0 + wn0 + 16 tj + sl, kk = k0 + wk0 +
  // 16 ti + 4 g.
#pragma unroll
  for (int tj = 0; tj < C::kTJ; ++tj) {
    const int nn = n0 + wn0 + 16 * tj + sl;
    if (nn >= n) continue;
    float* row = dw + static_cast<int64_t>(nn) * lddw;
#pragma unroll
    for (int ti = 0; ti < C::kTI; ++ti) {
      const int kk = k0 + wk0 + 16 * ti + 4 * g;
      f32x4_t v = acc[ti][tj];
      if (vec_ok && kk + 4 <= k) {
        f32x4_t* dst = reinterpret_cast<f32x4_t*>(row + kk);
        if (accumulate) v += *dst;
        *dst = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (kk + e < k) row[kk + e] = accumulate ? row[kk + e] + v[e] : v[e];
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// m == 0: the sum is empty; without accumulate dW is zero.
__global__ void dw_fill_zero(float* dw, int n, int k, int lddw) {
  const int64_t total = static_cast<int64_t>(n) * k;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = i / k;
    dw[r * lddw + (i - r * k)] = 0.0f;
  }
}

template <int TK, int TN>
hipError_t launch_dw_tiles(const uint16_t* dy, int64_t m, int64_t n, int64_t lddy,
                           const uint16_t* x, int64_t k, int64_t ldx, float* dw, int64_t lddw,
                           bool accumulate, hipStream_t stream) {
  const int64_t tiles_k = (k + TK - 1) / TK;
  const int64_t tiles = tiles_k * ((n + TN - 1) / TN);
  const int vec_ok = (reinterpret_cast<uintptr_t>(dw) % 16 == 0) && (lddw % 4 == 0);
  hipLaunchKernelGGL((gemm_dw_mfma<TK, TN>), dim3(static_cast<unsigned>(tiles)),
                     dim3(kDwThreads), 0, stream, dy, static_cast<int>(m), static_cast<int>(n),
                     static_cast<int>(lddy), x, static_cast<int>(k), static_cast<int>(ldx), dw,
                     static_cast<int>(lddw), accumulate ? 1 : 0, static_cast<int>(tiles_k),
                     vec_ok);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_dw(const uint16_t* dy, int64_t m, int64_t n, int64_t lddy,
                          const uint16_t* x, int64_t k, int64_t ldx, float* dw, int64_t lddw,
                          bool accumulate, hipStream_t stream) {
  if (m == 0) {
    if (accumulate) return hipSuccess;
    int64_t blocks = (n * k + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(dw_fill_zero, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, dw,
                       static_cast<int>(n), static_cast<int>(k), static_cast<int>(lddw));
    return hipGetLastError();
  }
  const int64_t big = ((k + 255) / 256) * ((n + 255) / 256);
  if (big >= 256)
    return launch_dw_tiles<256, 256>(dy, m, n, lddy, x, k, ldx, dw, lddw, accumulate, stream);
  return launch_dw_tiles<128, 128>(dy, m, n, lddy, x, k, ldx, dw, lddw, accumulate, stream);
}

}  // namespace tern
