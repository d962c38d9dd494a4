// Ternary linear layer: Y = bf16((X . T^T) (.) s), bf16 X, 2-bit packed T.
//
// "1.58-bit FLUX" (arXiv 2412.18653) builds an efficient linear kernel for
// 1.58-bit weights with unquantized activations (section 1 contributions,
// section 3.2, section 4 limitations).  At diffusion-transformer sequence
// lengths (thousands of tokens) this is a dense contraction, so it runs on
// the bf16 matrix cores of gfx950 with fp32 accumulation.
//
// Design (large M):
//  * Block tile 256 (X rows, "M") x 256 (weight rows, "N"), K step 64,
//    256 threads = 4 waves as 2 x 2, each wave owning 128 x 128 outputs as
//    4 x 4 tiles of v_mfma_f32_32x32x16_bf16.
//  * The weight matrix is the MFMA's A operand (rows = output channels) and
//    X is the B operand, so each lane ends up holding four consecutive output
//    channels of one token: the epilogue writes 8-byte runs of Y.
//  * Packed weights (4 KiB per block per K step) are staged through LDS
//    next to the X tile, then each lane reads the 8 bytes (32 codes) it needs
//    per 32-row tile and decodes them in registers.  With the 2-bit codes 00 / 01 / 11 the bf16 value code << 14
//    is exactly 0 / +2.0 / -2.0, so a decode is a byte permute, a shift and a
//    mask per pair of weights; the factor 2 is removed exactly in the
//    epilogue.
//  * X goes HBM -> registers -> LDS (double buffered, 16-byte chunks XOR
//    swizzled by row so that both the row-wise writes and the column-wise
//    MFMA reads are free of bank conflicts) and is read back with 16-byte LDS
//    loads.
//  * Epilogue: fp32 accumulator times the fp32 channel scale, one
//    round-to-nearest-even conversion to bf16, stored straight to HBM.
//  * Workgroups are renumbered so that each XCD (which owns its own L2)
//    walks a contiguous, grouped range of tiles.
//  * Ragged M and N edges: buffer loads past the valid rows return zeros and
//    the stores are predicated.  K must be a multiple of 64.
#include "internal.h"

namespace tern {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;

constexpr int kThreads = 256;
constexpr int kBM = 256;   // X rows per block
constexpr int kBN = 256;   // weight rows (output channels) per block
constexpr int kBK = 64;    // K per pipeline stage
constexpr int kTM = 4;     // 32-wide MFMA tiles per wave along M
constexpr int kTN = 4;     // 32-wide MFMA tiles per wave along N
constexpr int kXLoads = kBM * kBK * 2 / 16 / kThreads;  // 16-byte X loads per thread per stage
constexpr int kLdsX = kBM * kBK * 2;                    // X bytes of one stage in LDS
constexpr int kLdsStage = kLdsX + kBN * kBK / 4;        // X tile + packed weight tile
constexpr int kGroupM = 8;                              // M tiles per L2 group
constexpr uint32_t kRsrcWord3 = 0x00020000u;            // raw buffer, 32-bit data format

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), static_cast<int>(kRsrcWord3));
}

// Eight weights (codes of one lane, one MFMA k-block) -> eight bf16 values
// 0 / +2 / -2 in four registers, in ascending k.  `w` holds 16 codes; `hi`
// selects codes 8..15 instead of 0..7.  After the byte permute, half-word 0
// holds the selected codes in their original place and half-word 1 holds the
// same codes moved down by one field, so shifting left by 14 - 4q and masking
// leaves code 2q in bits 14..15 and code 2q+1 in bits 30..31.
__device__ inline bf16x8_t decode8(uint32_t w, bool hi) {
  const uint32_t w2 = w >> 2;
  const uint32_t h = __builtin_amdgcn_perm(w2, w, hi ? 0x07060302u : 0x05040100u);
  u32x4_t d;
  d[0] = (h << 14) & 0xC000C000u;
  d[1] = (h << 10) & 0xC000C000u;
  d[2] = (h << 6) & 0xC000C000u;
  d[3] = (h << 2) & 0xC000C000u;
  return __builtin_bit_cast(bf16x8_t, d);
}

// Maps the hardware workgroup id to a (tile_m, tile_n) pair.  Workgroups are
// dealt to the 8 XCDs round-robin; renumbering gives each XCD a contiguous
// block of the logical order, and the logical order visits tiles in groups
// of kGroupM M-tiles so that concurrently running tiles share X rows and
// weight rows in that XCD's L2.
__device__ inline void tile_of(int bid, int grid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int xcd = bid & 7;
  const int local = bid >> 3;
  const int per = grid >> 3;
  const int rem = grid & 7;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + local;
  const int in_group = kGroupM * tiles_n;
  const int group = logical / in_group;
  const int first_m = group * kGroupM;
  const int gsm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int r = logical - group * in_group;
  tm = first_m + r % gsm;
  tn = r / gsm;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_ternary_large(const uint16_t* __restrict__ x, int m, int k, int ldx,
                        const uint8_t* __restrict__ p, int n, int ldp,
                        const float* __restrict__ s, uint16_t* __restrict__ y, int ldy,
                        int tiles_m, int tiles_n, int y_vec_ok) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kLdsStage];

  int tile_m, tile_n;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tile_m, tile_n);
  const int m0 = tile_m * kBM;
  const int n0 = tile_n * kBN;
  const int rows_m = (m - m0) < kBM ? (m - m0) : kBM;
  const int rows_n = (n - n0) < kBN ? (n - n0) : kBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int l32 = lane & 31;
  const int lhi = lane >> 5;

  // Buffer resources rebased at this block's first row: reads past the last
  // valid row fall outside num_records and return zeros.
  const __amdgpu_buffer_rsrc_t x_rsrc =
      make_rsrc(x + static_cast<int64_t>(m0) * ldx,
                static_cast<uint32_t>((static_cast<int64_t>(rows_m - 1) * ldx + k) * 2));
  const __amdgpu_buffer_rsrc_t p_rsrc =
      make_rsrc(p + static_cast<int64_t>(n0) * ldp,
                static_cast<uint32_t>(static_cast<int64_t>(rows_n - 1) * ldp + k / 4));

  // X staging: thread -> (row, 16-byte chunk); rows tid/8 + 32 i.
  const int xc = tid & 7;
  const int xrow0 = tid >> 3;
  uint32_t x_voff[kXLoads];
  uint32_t x_lds[kXLoads];
#pragma unroll
  for (int i = 0; i < kXLoads; ++i) {
    const int r = xrow0 + 32 * i;
    x_voff[i] = (static_cast<uint32_t>(r) * static_cast<uint32_t>(ldx) + 8u * xc) * 2u;
    x_lds[i] = static_cast<uint32_t>(r * 128 + ((xc ^ (r & 7)) << 4));
  }
  // Weight-code staging: thread -> weight row tid, the 16-byte (64-code)
  // slice of the K step.
  const uint32_t p_voff = static_cast<uint32_t>(tid) * static_cast<uint32_t>(ldp);
  const uint32_t p_lds = kLdsX + static_cast<uint32_t>(tid) * 16u;
  // MFMA B-operand (X) reads: row (wm*128 + 32*i + l32), chunk 4*lhi + b.
  uint32_t xf_lds[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
    xf_lds[b] = static_cast<uint32_t>((wm * 128 + l32) * 128 + (((4 * lhi + b) ^ (l32 & 7)) << 4));
  // MFMA A-operand (weights) codes: row (wn*128 + 32*j + l32), bytes 8*lhi .. +7.
  const uint32_t pf_lds = kLdsX + static_cast<uint32_t>((wn * 128 + l32) * 16 + 8 * lhi);

  f32x16_t acc[kTN][kTM];
#pragma unroll
  for (int j = 0; j < kTN; ++j)
#pragma unroll
    for (int i = 0; i < kTM; ++i) acc[j][i] = f32x16_t{};

  const int stages = k / kBK;
  u32x4_t xreg[kXLoads];
  u32x4_t preg;

  auto load_stage = [&](int stage) {
#pragma unroll
    for (int i = 0; i < kXLoads; ++i)
      xreg[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                x_rsrc, x_voff[i], stage * kBK * 2, 0));
    preg = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                           p_rsrc, p_voff, stage * (kBK / 4), 0));
  };
  auto store_stage = [&](int buf) {
    uint8_t* base = lds + buf * kLdsStage;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) *reinterpret_cast<u32x4_t*>(base + x_lds[i]) = xreg[i];
    *reinterpret_cast<u32x4_t*>(base + p_lds) = preg;
  };

  // Pipeline: while step s computes out of one LDS buffer, the global loads
  // of step s+1 (issued one step earlier) land in registers; they are written
  // to the other buffer after the compute, and step s+2 is requested.
  load_stage(0);
  store_stage(0);
  if (stages > 1) load_stage(1);
  __syncthreads();
  for (int st = 0; st < stages; ++st) {
    const uint8_t* base = lds + (st & 1) * kLdsStage;
    u32x2_t pc[kTN];
#pragma unroll
    for (int j = 0; j < kTN; ++j)
      pc[j] = *reinterpret_cast<const u32x2_t*>(base + pf_lds + j * 32 * 16);
    // Four MFMA k-blocks of 16; in block b the lanes with lhi = h cover
    // k = 32 h + 8 b .. 32 h + 8 b + 7 of the step, for both operands.
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      bf16x8_t xf[kTM];
#pragma unroll
      for (int i = 0; i < kTM; ++i)
        xf[i] = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t*>(base + xf_lds[b] + i * 32 * 128));
      bf16x8_t wf[kTN];
#pragma unroll
      for (int j = 0; j < kTN; ++j) wf[j] = decode8(b < 2 ? pc[j][0] : pc[j][1], (b & 1) != 0);
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int i = 0; i < kTM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], xf[i], acc[j][i], 0, 0, 0);
    }
    if (st + 1 < stages) store_stage((st & 1) ^ 1);
    if (st + 2 < stages) load_stage(st + 2);
    __syncthreads();
  }

  // Epilogue.  Lane holds, for tile (j, i) and register r, output channel
  // n = 32 j + 8 (r / 4) + 4 lhi + (r % 4) and token m = 32 i + l32.  The
  // decode produced 2 T, so y = bf16(fp32(acc * s) * 0.5), which equals
  // bf16(fp32(acc / 2 * s)) exactly.
#pragma unroll
  for (int j = 0; j < kTN; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nl = wn * 128 + 32 * j + 8 * q + 4 * lhi;
      const int ng = n0 + nl;
      float sc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[e] = (ng + e < n) ? s[ng + e] : 0.0f;
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        const int mg = m0 + wm * 128 + 32 * i + l32;
        if (mg >= m) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (acc[j][i][4 * q + e] * sc[e]) * 0.5f;
        const __bf16 b0 = static_cast<__bf16>(v[0]);
        const __bf16 b1 = static_cast<__bf16>(v[1]);
        const __bf16 b2 = static_cast<__bf16>(v[2]);
        const __bf16 b3 = static_cast<__bf16>(v[3]);
        uint16_t* yr = y + static_cast<int64_t>(mg) * ldy + ng;
        if (y_vec_ok && ng + 4 <= n) {
          u32x2_t o;
          o[0] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b0)) |
                 (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b1)) << 16);
          o[1] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b2)) |
                 (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b3)) << 16);
          *reinterpret_cast<u32x2_t*>(yr) = o;
        } else {
          const __bf16 bb[4] = {b0, b1, b2, b3};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (ng + e < n) yr[e] = __builtin_bit_cast(uint16_t, bb[e]);
        }
      }
    }
  }
}

// k == 0: the sum is empty, so Y = bf16(0 * s) = 0.
__global__ void fill_zero_bf16(uint16_t* y, int m, int n, int ldy) {
  const int64_t total = static_cast<int64_t>(m) * n;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = i / n;
    y[r * ldy + (i - r * n)] = 0;
  }
}

}  // namespace

hipError_t launch_gemm(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const uint8_t* p,
                       int64_t n, int64_t ldp, const float* s, uint16_t* y, int64_t ldy,
                       hipStream_t stream) {
  if (k == 0) {
    int64_t blocks = (m * n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_zero_bf16, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       y, static_cast<int>(m), static_cast<int>(n), static_cast<int>(ldy));
    return hipGetLastError();
  }
  const int tiles_m = static_cast<int>((m + kBM - 1) / kBM);
  const int tiles_n = static_cast<int>((n + kBN - 1) / kBN);
  const int y_vec_ok = ((reinterpret_cast<uintptr_t>(y) & 7) == 0) && (ldy % 4 == 0);
  hipLaunchKernelGGL(gemm_ternary_large, dim3(static_cast<unsigned>(tiles_m) * tiles_n),
                     dim3(kThreads), 0, stream, x, static_cast<int>(m), static_cast<int>(k),
                     static_cast<int>(ldx), p, static_cast<int>(n), static_cast<int>(ldp), s, y,
                     static_cast<int>(ldy), tiles_m, tiles_n, y_vec_ok);
  return hipGetLastError();
}

}  // namespace tern
