// Ternary linear layer: Y = bf16((X . T^T) (.) s), bf16 X, 2-bit packed T.
//
// "1.58-bit FLUX" (arXiv 2412.18653) builds an efficient linear kernel for
// 1.58-bit weights with unquantized activations (section 1 contributions,
// section 3.2, section 4 limitations).  At diffusion-transformer sequence
// lengths (thousands of tokens) this is a dense contraction, so it runs on
// the bf16 matrix cores of gfx950 with fp32 accumulation.
//
// Design:
//  * Block tile BM (X rows, "M") x BN (weight rows = output channels, "N"),
//    K step 64, 256 threads = 4 waves as 2 x 2.  Each wave owns
//    (BM/2) x (BN/2) outputs as 16 x 16 tiles of v_mfma_f32_16x16x32_bf16.
//    288 x 192 divides M = 4608 and every FLUX width N into a multiple of
//    256 blocks, so all 256 CUs stay busy to the last block.
//  * The weight tile is the MFMA's A operand and X the B operand, so every
//    lane ends up with four consecutive output channels of one token and the
//    epilogue writes 8-byte runs of Y.
//  * Operands reach LDS without passing through registers: buffer loads with
//    the LDS-DMA form (16 bytes per lane) fill a 3-stage ring, so the loads
//    of step s+2 are in flight while step s computes.  Loads past the last
//    valid row of X or of the weights return zeros (buffer range checking).
//  * X rows are 128 bytes per stage, stored as 16-byte chunks XOR-swizzled
//    by (row & 7); the swizzle is applied on the global side (each lane
//    fetches the chunk that belongs in its LDS slot), so the MFMA operand
//    reads (one 16-byte chunk per lane, 16 rows at a time) hit 8 distinct
//    bank groups.
//  * The packed weights stay packed in LDS (16 bytes = 64 codes per row per
//    step).  Each lane reads one 32-bit word (16 codes) per 16-row tile and
//    decodes it in registers: with codes 00 / 01 / 11 the bf16 value
//    code << 14 is exactly 0 / +2.0 / -2.0, so two weights cost a shift and
//    a mask after one byte permute.  The factor 2 is removed exactly in the
//    epilogue.
//  * Epilogue: fp32 accumulator times the fp32 channel scale, one
//    round-to-nearest-even conversion to bf16.
//  * Workgroups are renumbered so that each XCD (which owns its own L2)
//    walks a contiguous, grouped range of tiles.
#include "internal.h"

namespace tern {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kThreads = 256;
constexpr int kBK = 64;                       // K per pipeline stage
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), static_cast<int>(kRsrcWord3));
}

// s_waitcnt for this wave: vector-memory counter <= N and, with LGKM0, all
// LDS operations complete.  (lgkmcnt saturates at 15 outstanding operations:
// keeping at most one batch of operand reads in flight lets the compiler's
// own waits stay exact.)
template <int N, bool LGKM0 = false>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | ((LGKM0 ? 0 : 15) << 8));
}
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Pins the schedule at a phase boundary: no memory access (compiler level)
// and no instruction at all (machine scheduler) moves across it.
__device__ inline void phase_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier that orders LDS accesses for the compiler without a
// memory fence: the fence of __syncthreads() would also wait for every DMA in
// flight, which defeats the ring.  The empty asm statements with a memory
// clobber keep the compiler from moving any load or store across the barrier;
// visibility of the DMA writes is established by the vmcnt wait each wave
// performs before arriving.
__device__ inline void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Sixteen 2-bit codes -> two MFMA operands of eight bf16 values (0 / +2 / -2)
// in ascending k: `lo` gets codes 0..7, `hi` codes 8..15.  After the byte
// permute, half-word 0 holds the selected codes in place and half-word 1 the
// same codes moved down one field, so a left shift by 14 - 4q and a mask
// leave code 2q in bits 14..15 and code 2q+1 in bits 30..31.
__device__ inline void decode16(uint32_t w, bf16x8_t& lo, bf16x8_t& hi) {
  const uint32_t w2 = w >> 2;
  const uint32_t h0 = __builtin_amdgcn_perm(w2, w, 0x05040100u);
  const uint32_t h1 = __builtin_amdgcn_perm(w2, w, 0x07060302u);
  u32x4_t a, b;
  a[0] = (h0 << 14) & 0xC000C000u;
  a[1] = (h0 << 10) & 0xC000C000u;
  a[2] = (h0 << 6) & 0xC000C000u;
  a[3] = (h0 << 2) & 0xC000C000u;
  b[0] = (h1 << 14) & 0xC000C000u;
  b[1] = (h1 << 10) & 0xC000C000u;
  b[2] = (h1 << 6) & 0xC000C000u;
  b[3] = (h1 << 2) & 0xC000C000u;
  lo = __builtin_bit_cast(bf16x8_t, a);
  hi = __builtin_bit_cast(bf16x8_t, b);
}

// Maps the hardware workgroup id to a (tile_m, tile_n) pair.  Workgroups are
// dealt to the 8 XCDs round-robin; renumbering gives each XCD a contiguous
// block of the logical order, and the logical order visits tiles in groups
// of GM M-tiles so that concurrently running tiles share X rows and weight
// rows in that XCD's L2.
template <int GM>
__device__ inline void tile_of(int bid, int grid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int xcd = bid & 7;
  const int local = bid >> 3;
  const int per = grid >> 3;
  const int rem = grid & 7;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + local;
  const int in_group = GM * tiles_n;
  const int group = logical / in_group;
  const int first_m = group * GM;
  const int gsm = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int r = logical - group * in_group;
  tm = first_m + r % gsm;
  tn = r / gsm;
}

// X chunk swizzle of LDS row r: the 16-byte chunk c of a row is stored in
// slot c ^ xswz(r).
template <int SWZ>
__device__ inline uint32_t xswz(uint32_t r) {
  return SWZ == 0 ? (r & 7u) : ((r >> 1) & 7u);
}

template <int BM, int BN, int WAVES_M>
struct TileCfg {
  static constexpr int kWavesM = WAVES_M;          // waves along M
  static constexpr int kWavesN = 4 / WAVES_M;      // waves along N
  static constexpr int kWM = BM / kWavesM;         // wave tile rows (M)
  static constexpr int kWN = BN / kWavesN;         // wave tile rows (N)
  static constexpr int kTM = kWM / 16;             // 16x16 MFMA tiles per wave along M
  static constexpr int kTN = kWN / 16;             // ... along N
  static constexpr int kXBytes = BM * kBK * 2;     // X bytes per stage (128 per row)
  static constexpr int kPBytes = BN * kBK / 4;     // packed weight bytes per stage (16 per row)
  static constexpr int kStage = kXBytes + kPBytes;
  static constexpr int kXInstr = kXBytes / 1024;   // 1 KiB DMA instructions per stage: X
  static constexpr int kPInstr = kPBytes / 1024;   // ... packed weights
  static constexpr int kLoads = (kXInstr + kPInstr) / 4;  // per wave per stage
  static_assert(WAVES_M == 1 || WAVES_M == 2 || WAVES_M == 4, "4 waves");
  static_assert(kWM % 16 == 0 && kWN % 16 == 0, "whole MFMA tiles");
  static_assert(BM % 8 == 0 && BN % 64 == 0, "whole DMA instructions");
  static_assert((kXInstr + kPInstr) % 4 == 0, "same DMA count on every wave");
  static_assert((kWM * 128) % 1024 == 0 || kWavesM == 1, "row swizzle period");
};

template <int BM, int BN, int WAVES_M, int GM, int SWZ>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_ternary_mfma(const uint16_t* __restrict__ x, int m, int k, int ldx,
                       const uint8_t* __restrict__ p, int n, int ldp,
                       const float* __restrict__ s, uint16_t* __restrict__ y, int ldy,
                       int tiles_m, int tiles_n, int y_vec_ok) {
#if defined(__HIP_DEVICE_COMPILE__)
  // (The body uses LDS address-space casts that only the device pass accepts.)
  using C = TileCfg<BM, BN, WAVES_M>;
  constexpr int kTM = C::kTM;
  constexpr int kTN = C::kTN;
  // One LDS object per ring stage, so that the compiler tracks each stage's
  // DMA writes separately.  kRing = 6 stages: one being read, one being read
  // next, four in flight (the DMA stream is latency-bound, so the bytes in
  // flight set its rate).
  constexpr int kRing = 6;
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds4[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds5[C::kStage];

  int tile_m, tile_n;
  tile_of<GM>(blockIdx.x, gridDim.x, tiles_m, tiles_n, tile_m, tile_n);
  const int m0 = tile_m * BM;
  const int n0 = tile_n * BN;
  const int rows_m = (m - m0) < BM ? (m - m0) : BM;
  const int rows_n = (n - n0) < BN ? (n - n0) : BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % C::kWavesM;
  const int wn = wave / C::kWavesM;
  const int l16 = lane & 15;
  const int g = lane >> 4;  // k-group of the MFMA operands

  const __amdgpu_buffer_rsrc_t x_rsrc =
      make_rsrc(x + static_cast<int64_t>(m0) * ldx,
                static_cast<uint32_t>((static_cast<int64_t>(rows_m - 1) * ldx + k) * 2));
  const __amdgpu_buffer_rsrc_t p_rsrc =
      make_rsrc(p + static_cast<int64_t>(n0) * ldp,
                static_cast<uint32_t>(static_cast<int64_t>(rows_n - 1) * ldp + k / 4));

  // DMA plan.  A stage is kXInstr + kPInstr loads of 1 KiB (16 bytes per
  // lane); wave w issues loads w, w+4, w+8, ... in that list.  X load q fills
  // LDS bytes [1024 q, +1024): rows 8 q + lane/8, slot lane%8, which holds
  // logical chunk (lane%8) ^ xswz(row).  Weight load p fills [kXBytes +
  // 1024 p, +1024): rows 64 p + lane, 16 bytes each.
  uint32_t dma_voff[C::kLoads];
  uint32_t dma_lds[C::kLoads];
  bool dma_is_x[C::kLoads];
#pragma unroll
  for (int q = 0; q < C::kLoads; ++q) {
    const int gi = wave + 4 * q;
    dma_is_x[q] = gi < C::kXInstr;
    if (dma_is_x[q]) {
      const uint32_t r = 8u * gi + (lane >> 3);
      const uint32_t c = (lane & 7) ^ xswz<SWZ>(r);
      dma_voff[q] = (r * static_cast<uint32_t>(ldx) + 8u * c) * 2u;
      dma_lds[q] = 1024u * gi;
    } else {
      const uint32_t r = 64u * (gi - C::kXInstr) + lane;
      dma_voff[q] = r * static_cast<uint32_t>(ldp);
      dma_lds[q] = C::kXBytes + 1024u * (gi - C::kXInstr);
    }
  }

  // Requests step `stage` into ring stage BUF (one of the lds* arrays, named
  // directly so that the compiler can tell the stages apart).
#define TERN_GEMM_DMA(BUF, STAGE, Q)                                                   \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(dma_is_x[Q] ? x_rsrc : p_rsrc,               \
                                           (lds_void_t*)(&BUF[dma_lds[Q]]), 16,        \
                                           dma_voff[Q],                                \
                                           (STAGE) * (dma_is_x[Q] ? kBK * 2 : kBK / 4), 0, 0);
#define TERN_GEMM_ISSUE(BUF, STAGE) \
  _Pragma("unroll") for (int q = 0; q < C::kLoads; ++q) TERN_GEMM_DMA(BUF, STAGE, q)

  // MFMA operand reads.  Block b of a step covers, for the lanes of k-group
  // g, k = 16 g + 8 b .. 16 g + 8 b + 7 of the step: X chunk 2 g + b of row
  // (wm*kWM + 16 i + l16), and codes 8 b .. 8 b + 7 of 32-bit word g of
  // weight row (wn*kWN + 16 j + l16).
  const uint32_t x_row0 = static_cast<uint32_t>(wm * C::kWM + l16);
  const uint32_t xo0 = x_row0 * 128u + ((static_cast<uint32_t>(2 * g + 0) ^ xswz<SWZ>(x_row0)) << 4);
  const uint32_t xo1 = x_row0 * 128u + ((static_cast<uint32_t>(2 * g + 1) ^ xswz<SWZ>(x_row0)) << 4);
  const uint32_t po = C::kXBytes + static_cast<uint32_t>(wn * C::kWN + l16) * 16u + 4u * g;

  f32x4_t acc[kTN][kTM];
#pragma unroll
  for (int j = 0; j < kTN; ++j)
#pragma unroll
    for (int i = 0; i < kTM; ++i) acc[j][i] = f32x4_t{};

  // Operand reads out of ring stage BUF (named directly, see above): the
  // 32-bit code words of every weight tile and the X chunks of k-block 0
  // (READ_A), or the X chunks of k-block 1 (READ_B).
#define TERN_GEMM_READ_A(BUF)                                                               \
  _Pragma("unroll") for (int j = 0; j < kTN; ++j)                                           \
      pw[j] = *reinterpret_cast<const uint32_t*>(&BUF[po + j * 256]);                       \
  _Pragma("unroll") for (int i = 0; i < kTM; ++i)                                           \
      xa[i] = __builtin_bit_cast(bf16x8_t,                                                  \
                                 *reinterpret_cast<const u32x4_t*>(&BUF[xo0 + i * 2048]));
#define TERN_GEMM_READ_B(BUF)                                                               \
  _Pragma("unroll") for (int i = 0; i < kTM; ++i)                                           \
      xb[i] = __builtin_bit_cast(bf16x8_t,                                                  \
                                 *reinterpret_cast<const u32x4_t*>(&BUF[xo1 + i * 2048]));

  auto mfma_block = [&](const bf16x8_t (&w)[kTN], const bf16x8_t (&xv)[kTM]) {
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int i = 0; i < kTM; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[j], xv[i], acc[j][i], 0, 0, 0);
  };

  // Scheduling hint for the phase after the barrier: spread the DMA requests
  // and the operand reads of the next stage between the MFMAs instead of
  // issuing them back to back (a stalled memory instruction would hold up the
  // MFMAs behind it).
  auto interleave_loads_with_mfma = [&]() {
    constexpr int kReads = kTM + (kTN + 1) / 2;   // ds_read instructions of READ_A
    constexpr int kGroups = C::kLoads;
    constexpr int kMfma = kTN * kTM;
#pragma unroll
    for (int i = 0; i < kGroups; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x0010, 1, 0);                       // DMA
      __builtin_amdgcn_sched_group_barrier(0x0100, (kReads + kGroups - 1) / kGroups, 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x0008, kMfma / kGroups, 0);         // MFMA
    }
  };

  // Step ST computes out of ring stage CUR.  Its k-block 0 operands were read
  // during the previous step.  It reads k-block 1 and runs k-block 0; then,
  // once every wave is past the barrier (so stage ST+1 has landed everywhere
  // and stage ST-1 is no longer read by anyone), it requests stage
  // ST+kRing-1 into ST-1's buffer DMA, reads stage ST+1's k-block 0 out of NXT, and runs
  // k-block 1.  LDS serves each batch of reads while the other k-block's
  // MFMAs run, and at most one batch is outstanding at any time.
  //
  // The main loop keeps exactly kRing-2 stages in flight at every barrier: a
  // request past the last stage re-loads the last stage into the dead buffer
  // (in range, never read), so that every step issues the same instructions
  // and the compiler's wait counts stay exact.  The last one to four steps
  // run in a tail with the waits shortened accordingly.
  const int stages = k / kBK;
#define TERN_GEMM_STAGE(S) ((S) < stages ? (S) : stages - 1)
#define TERN_GEMM_HALF_A(CUR)                                      \
  phase_fence();                                                   \
  wait_lgkm0();                                                    \
  TERN_GEMM_READ_B(CUR)                                            \
  phase_fence();                                                   \
  bf16x8_t wa[kTN], wb[kTN];                                       \
  _Pragma("unroll") for (int j = 0; j < kTN; ++j) decode16(pw[j], wa[j], wb[j]); \
  mfma_block(wa, xa);                                              \
  phase_fence();                                                   \
  wait_lgkm0();
#define TERN_GEMM_STEP(ST, CUR, NXT, DMA)                          \
  {                                                                \
    TERN_GEMM_HALF_A(CUR)                                          \
    wait_vmcnt<(kRing - 3) * C::kLoads, true>();                   \
    lds_barrier();                                                 \
    TERN_GEMM_ISSUE(DMA, TERN_GEMM_STAGE((ST) + kRing - 1))        \
    TERN_GEMM_READ_A(NXT)                                          \
    mfma_block(wb, xb);                                            \
    interleave_loads_with_mfma();                                  \
  }
  // Tail step: requests stage ST+kRing-1 if it exists (only the first tail step
  // can have one), waits for everything in flight, and reads the next stage
  // if there is one.
#define TERN_GEMM_TAIL(ST, CUR, NXT, DMA)                          \
  {                                                                \
    TERN_GEMM_HALF_A(CUR)                                          \
    if ((ST) + 1 < stages) {                                       \
      wait_vmcnt<0, true>();                                       \
      lds_barrier();                                               \
      if ((ST) + kRing - 1 < stages) TERN_GEMM_ISSUE(DMA, (ST) + kRing - 1) \
      TERN_GEMM_READ_A(NXT)                                        \
      phase_fence();                                               \
    }                                                              \
    mfma_block(wb, xb);                                            \
  }
  uint32_t pw[kTN];
  bf16x8_t xa[kTM], xb[kTM];
  TERN_GEMM_ISSUE(lds0, 0)
  TERN_GEMM_ISSUE(lds1, TERN_GEMM_STAGE(1))
  TERN_GEMM_ISSUE(lds2, TERN_GEMM_STAGE(2))
  TERN_GEMM_ISSUE(lds3, TERN_GEMM_STAGE(3))
  TERN_GEMM_ISSUE(lds4, TERN_GEMM_STAGE(4))
  wait_vmcnt<(kRing - 2) * C::kLoads, true>();
  lds_barrier();
  TERN_GEMM_READ_A(lds0)
  int st = 0;
  for (; st + kRing < stages; st += kRing) {
    TERN_GEMM_STEP(st, lds0, lds1, lds5)
    TERN_GEMM_STEP(st + 1, lds1, lds2, lds0)
    TERN_GEMM_STEP(st + 2, lds2, lds3, lds1)
    TERN_GEMM_STEP(st + 3, lds3, lds4, lds2)
    TERN_GEMM_STEP(st + 4, lds4, lds5, lds3)
    TERN_GEMM_STEP(st + 5, lds5, lds0, lds4)
  }
  // 1 to kRing steps remain, starting at ring stage 0.
  TERN_GEMM_TAIL(st, lds0, lds1, lds5)
  if (st + 1 < stages) TERN_GEMM_TAIL(st + 1, lds1, lds2, lds0)
  if (st + 2 < stages) TERN_GEMM_TAIL(st + 2, lds2, lds3, lds1)
  if (st + 3 < stages) TERN_GEMM_TAIL(st + 3, lds3, lds4, lds2)
  if (st + 4 < stages) TERN_GEMM_TAIL(st + 4, lds4, lds5, lds3)
  if (st + 5 < stages) TERN_GEMM_TAIL(st + 5, lds5, lds0, lds4)
  wait_vmcnt<0>();  // no DMA may outlive the workgroup's LDS
#undef TERN_GEMM_STEP
#undef TERN_GEMM_TAIL
#undef TERN_GEMM_HALF_A
#undef TERN_GEMM_STAGE
#undef TERN_GEMM_ISSUE
#undef TERN_GEMM_DMA
#undef TERN_GEMM_READ_A
#undef TERN_GEMM_READ_B

  // Epilogue.  For tile (j, i) the lane holds output channels
  // n = wn*kWN + 16 j + 4 g + e (e = 0..3) of token m = wm*kWM + 16 i + l16.
  // The decode produced 2 T, so y = bf16(fp32(acc * s) * 0.5), which equals
  // bf16(fp32(acc / 2 * s)) exactly.
#pragma unroll
  for (int j = 0; j < kTN; ++j) {
    const int ng = n0 + wn * C::kWN + 16 * j + 4 * g;
    float sc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) sc[e] = (ng + e < n) ? s[ng + e] : 0.0f;
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int mg = m0 + wm * C::kWM + 16 * i + l16;
      if (mg >= m) continue;
      __bf16 b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) b[e] = static_cast<__bf16>((acc[j][i][e] * sc[e]) * 0.5f);
      uint16_t* yr = y + static_cast<int64_t>(mg) * ldy + ng;
      if (y_vec_ok && ng + 4 <= n) {
        u32x2_t o;
        o[0] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b[0])) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b[1])) << 16);
        o[1] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b[2])) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b[3])) << 16);
        *reinterpret_cast<u32x2_t*>(yr) = o;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (ng + e < n) yr[e] = __builtin_bit_cast(uint16_t, b[e]);
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
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

template <int BM, int BN, int WAVES_M, int GM, int SWZ>
hipError_t launch_tiles(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const uint8_t* p,
                        int64_t n, int64_t ldp, const float* s, uint16_t* y, int64_t ldy,
                        hipStream_t stream) {
  const int tiles_m = static_cast<int>((m + BM - 1) / BM);
  const int tiles_n = static_cast<int>((n + BN - 1) / BN);
  const int y_vec_ok = ((reinterpret_cast<uintptr_t>(y) & 7) == 0) && (ldy % 4 == 0);
  hipLaunchKernelGGL((gemm_ternary_mfma<BM, BN, WAVES_M, GM, SWZ>),
                     dim3(static_cast<unsigned>(tiles_m) * static_cast<unsigned>(tiles_n)),
                     dim3(kThreads), 0, stream, x, static_cast<int>(m), static_cast<int>(k),
                     static_cast<int>(ldx), p, static_cast<int>(n), static_cast<int>(ldp), s, y,
                     static_cast<int>(ldy), tiles_m, tiles_n, y_vec_ok);
  return hipGetLastError();
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
#ifndef TERN_GEMM_SWZ
#define TERN_GEMM_SWZ 0
#endif
  return launch_tiles<144, 384, 1, 4, TERN_GEMM_SWZ>(x, m, k, ldx, p, n, ldp, s, y, ldy, stream);
}

}  // namespace tern
