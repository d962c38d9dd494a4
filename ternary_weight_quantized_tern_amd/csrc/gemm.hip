// Ternary linear layer: Y = bf16((X . T^T) (.) s), bf16 X, 2-bit packed T.
//
// "1.58-bit FLUX" (arXiv 2412.18653) builds an efficient linear kernel for
// 1.58-bit weights with unquantized activations (section 1 contributions,
// section 3.2, section 4 limitations).  At diffusion-transformer sequence
// lengths (thousands of tokens) this is a dense contraction, so it runs on
// the bf16 matrix cores of gfx950 with fp32 accumulation.
//
// Design:
//  * Block tile 144 (X rows, "M") x 384 (weight rows = output channels, "N"),
//    K step 64, 256 threads = 4 waves side by side along N.  Each wave owns
//    144 x 96 outputs as 9 x 6 tiles of v_mfma_f32_16x16x32_bf16 (216
//    accumulator registers).  144 x 384 cuts M = 4608 and every FLUX width N
//    (3072, 9216, 12288, 15360, 21504) into an exact multiple of 256 tiles.
//  * The weight tile is the MFMA's A operand and X the B operand, so every
//    lane ends up with four consecutive output channels of one token and the
//    epilogue writes 8-byte runs of Y.
//  * Operands reach LDS without passing through registers: buffer loads in
//    the LDS-DMA form (16 bytes per lane) fill a 6-stage ring, four stages in
//    flight while one is computed and the next one's operands are read.  Loads
//    past the last valid row of X or of the weights return zeros (buffer
//    range checking).  One barrier per K step, in its middle: the second half
//    of the MFMAs covers the LDS reads of the next step and the DMA requests.
//  * X rows are 128 bytes per stage, stored as 16-byte chunks XOR-swizzled
//    by ((row >> 1) & 7); the swizzle is applied on the global side (each lane
//    fetches the chunk that belongs in its LDS slot), so the MFMA operand
//    reads (one 16-byte chunk per lane, 16 rows at a time) are free of bank
//    conflicts.
//  * The packed weights stay packed in LDS (16 bytes = 64 codes per row per
//    step).  Each lane reads one 32-bit word (16 codes) per 16-row tile and
//    decodes it in registers: with codes 00 / 01 / 11 the bf16 value
//    code << 14 is exactly 0 / +2.0 / -2.0.  Four shift-and-mask vectors
//    put every code in the top bits of a byte, and one byte permute per
//    operand register places two of them: 15 VALU instructions per 16
//    weights.  The factor 2 is removed exactly in the epilogue.
//  * Epilogue: fp32 accumulator times the fp32 channel scale, one
//    round-to-nearest-even conversion to bf16.
//  * Workgroups are renumbered so that each XCD (which owns its own L2)
//    walks a contiguous, grouped range of tiles.  When there are more tiles
//    than CUs and K / 64 is a multiple of 6, 256 persistent workgroups walk
//    the tiles with one unbroken DMA stream, hiding each tile's start-up
//    latency behind the previous tile's last steps.
//
// The same kernel, with its A8 flag, is the layer on int8 activations (the
// 8-bit-activation variant that "1.58-bit FLUX", section 4, names as the
// missing piece for latency): v_mfma_i32_16x16x64_i8 takes 16 int8 values
// per lane and operand where the bf16 instruction takes 8 bf16 values, so a
// stage holds K = 128 with the same 128-byte X rows and 32-byte weight rows.
// The weights come field-transposed (act.hip), which makes one shift and one
// mask per operand register the whole decode; the exact int32 sums are
// scaled by s[n] / 64 and the token's scale xs[m] in the epilogue.  Tiles
// 144 x 384 in a four-stage ring (30 KiB stages), 64 x 576, 144 x 256 or
// 64 x 128.
#include <type_traits>

#include "gemm_common.h"
#include "internal.h"

namespace tern {
namespace {

constexpr int kThreads = 256;
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

// Two fp32 values rounded to bf16 (nearest even) in one 32-bit word, the
// first in the low half (one v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// X chunk swizzle of LDS row r: the 16-byte chunk c of a 128-byte row is
// stored in slot c ^ xswz(r).  Two rows share one 256-byte line of the 64
// LDS banks; with ((r >> 1) & 7) the 16 rows that one 16-lane group of an
// operand read touches (same logical chunk) land in 16 distinct 16-byte bank
// groups, so a ds_read_b128 of 64 lanes takes the minimum four passes.
__device__ inline uint32_t xswz(uint32_t r) { return (r >> 1) & 7u; }

// A8: int8 activations (one byte per element) with the int8 matrix cores
// (v_mfma_i32_16x16x64_i8, K = 128 per stage); otherwise bf16 activations
// with the bf16 matrix cores (K = 64 per stage).  An X row is 128 bytes of a
// stage either way; a weight row is 16 bytes (64 codes) or 32 bytes (128).
template <int BM, int BN, int WAVES_M, bool A8>
struct TileCfg {
  static constexpr int kWavesM = WAVES_M;          // waves along M
  static constexpr int kWavesN = 4 / WAVES_M;      // waves along N
  static constexpr int kWM = BM / kWavesM;         // wave tile rows (M)
  static constexpr int kWN = BN / kWavesN;         // wave tile rows (N)
  static constexpr int kTM = kWM / 16;             // 16x16 MFMA tiles per wave along M
  static constexpr int kTN = kWN / 16;             // ... along N
  static constexpr int kXElem = A8 ? 1 : 2;        // bytes per X element
  static constexpr int kBK = A8 ? 128 : 64;        // K per pipeline stage
  static constexpr int kPRow = kBK / 4;            // packed weight bytes per row per stage
  static constexpr int kXBytes = BM * 128;         // X bytes per stage (128 per row)
  static constexpr int kPBytes = BN * kPRow;       // packed weight bytes per stage
  static constexpr int kStage = kXBytes + kPBytes;
  static constexpr int kXInstr = kXBytes / 1024;   // 1 KiB DMA instructions per stage: X
  static constexpr int kPInstr = kPBytes / 1024;   // ... packed weights
  static constexpr int kInstr = kXInstr + kPInstr;
  static constexpr int kLoads = (kInstr + 3) / 4;  // per wave per stage (the last ones may
                                                   // repeat load 0 to even the count)
  static_assert(WAVES_M == 1 || WAVES_M == 2 || WAVES_M == 4, "4 waves");
  static_assert(kWM % 16 == 0 && kWN % 16 == 0, "whole MFMA tiles");
  static_assert(BM % 8 == 0 && BN % 64 == 0, "whole DMA instructions");
  static_assert((kWM * 128) % 1024 == 0 || kWavesM == 1, "row swizzle period");
};

// Y tile kernel (A8: int8 X with a per-row scale xs, weights in the
// field-transposed packing; otherwise bf16 X, xs not read).  With PERSIST, workgroup b computes tiles b, b + G, b + 2G,
// ... of the XCD-aware order (G = gridDim.x, a multiple of 8, so that all of
// a workgroup's tiles stay on its XCD), and the K steps of consecutive tiles
// form one stream through the LDS ring: the requests run kRing-1 steps ahead
// of the MFMAs and cross into the next tile, so a tile's first stages are in
// LDS by the time the previous tile's epilogue ends.  Tile boundaries must
// fall between iterations of the kRing-step unrolled loop: PERSIST requires
// (k / kBK) % kRing == 0.  Without PERSIST each workgroup computes tile b
// only, for any k that is a multiple of 64 (128 with A8).  With EPI the epilogue adds
// bias[n] (when bias is not null) and applies the tanh-form GELU to columns
// n >= act_from; without it, bias and act_from are not read.
template <int BM, int BN, int WAVES_M, int GM, bool PERSIST, int WPE, bool EPI, bool A8,
          int RING = 6>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void gemm_ternary_mfma(const uint8_t* __restrict__ x, int m, int k, int ldx,
                       const float* __restrict__ xs, const uint8_t* __restrict__ p, int n, int ldp,
                       const float* __restrict__ s, const float* __restrict__ bias, int act_from,
                       uint16_t* __restrict__ y, int ldy, int tiles_m, int tiles_n, int y_flags) {
#if defined(__HIP_DEVICE_COMPILE__)
  // (The body uses LDS address-space casts that only the device pass accepts.)
  using C = TileCfg<BM, BN, WAVES_M, A8>;
  constexpr int kTM = C::kTM;
  constexpr int kTN = C::kTN;
  const int ldxb = ldx * C::kXElem;  // X pitch in bytes (< 2^24, checked by the host)
  // One LDS object per ring stage, so that the compiler tracks each stage's
  // DMA writes separately.  kRing = 6 stages: one being read, one being read
  // next, four in flight; or 4 (two in flight) where a stage is too large for
  // six (the int8 144 x 384 tile: 30 KiB per stage).
  constexpr int kRing = RING;
  static_assert(RING == 6 || RING == 4, "ring of 6 or 4 stages");
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds4[RING == 6 ? C::kStage : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t lds5[RING == 6 ? C::kStage : 1];

  const int num_tiles = tiles_m * tiles_n;
  const int grid = gridDim.x;
  const int bid = blockIdx.x;
  const int my_tiles = PERSIST ? (num_tiles - bid + grid - 1) / grid : 1;
  const int stages = k / C::kBK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < kThreads / 64);  // lets DMA slots 0-3 and 5 fold
  const int wm = wave % C::kWavesM;
  const int wn = wave / C::kWavesM;
  const int l16 = lane & 15;
  const int g = lane >> 4;  // k-group of the MFMA operands

  // Tile coordinates and buffer resources of this workgroup's t-th tile.
  // The resources are rebased at the tile's first row: reads past its last
  // valid row fall outside num_records and return zeros.
  auto tile_coords = [&](int t, int& m0, int& n0) {
    int tm, tn;
    tile_of<GM>(bid + t * grid, num_tiles, tiles_m, tiles_n, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
  };
  auto tile_rsrc = [&](int t, __amdgpu_buffer_rsrc_t& xr, __amdgpu_buffer_rsrc_t& pr) {
    int m0, n0;
    tile_coords(t, m0, n0);
    const int rows_m = (m - m0) < BM ? (m - m0) : BM;
    const int rows_n = (n - n0) < BN ? (n - n0) : BN;
    xr = make_rsrc(x + static_cast<int64_t>(m0) * ldxb,
                   static_cast<uint32_t>(static_cast<int64_t>(rows_m - 1) * ldxb +
                                         static_cast<int64_t>(k) * C::kXElem));
    pr = make_rsrc(p + static_cast<int64_t>(n0) * ldp,
                   static_cast<uint32_t>(static_cast<int64_t>(rows_n - 1) * ldp + k / 4));
  };

  // DMA plan.  A stage is kXInstr + kPInstr loads of 1 KiB (16 bytes per
  // lane); wave w issues loads w, w+4, w+8, ... in that list, every wave the
  // same number of them.  X load q fills
  // LDS bytes [1024 q, +1024): rows 8 q + lane/8, slot lane%8, which holds
  // logical chunk (lane%8) ^ xswz(row).  Weight load p fills [kXBytes +
  // 1024 p, +1024): rows 64 p + lane, 16 bytes each (A8: rows 32 p + lane/2,
  // half lane%2 of their 32 bytes).
  uint32_t dma_voff[C::kLoads];
  uint32_t dma_lds[C::kLoads];
  bool dma_is_x[C::kLoads];
#pragma unroll
  for (int q = 0; q < C::kLoads; ++q) {
    // A slot past the last load repeats load 0 (same bytes to the same place).
    const int gi = (wave + 4 * q) < C::kInstr ? wave + 4 * q : 0;
    dma_is_x[q] = gi < C::kXInstr;
    if (dma_is_x[q]) {
      const uint32_t r = 8u * gi + (lane >> 3);
      const uint32_t c = (lane & 7) ^ xswz(r);
      dma_voff[q] = r * static_cast<uint32_t>(ldxb) + 16u * c;
      dma_lds[q] = 1024u * gi;
    } else if constexpr (A8) {
      const uint32_t r = 32u * (gi - C::kXInstr) + (lane >> 1);
      dma_voff[q] = r * static_cast<uint32_t>(ldp) + 16u * (lane & 1);
      dma_lds[q] = C::kXBytes + 1024u * (gi - C::kXInstr);
    } else {
      const uint32_t r = 64u * (gi - C::kXInstr) + lane;
      dma_voff[q] = r * static_cast<uint32_t>(ldp);
      dma_lds[q] = C::kXBytes + 1024u * (gi - C::kXInstr);
    }
  }

  // Requests one step (stage STAGE of the tile whose resources are XR, PR)
  // into ring stage BUF, one of the lds* arrays, named directly so that the
  // compiler can tell the ring stages apart.  A stage past the end of K is
  // requested through an empty buffer resource and arrives as zeros, so every
  // iteration of the unrolled loop issues the same instructions (the wait
  // counts stay exact) and steps past the end add nothing.
  const __amdgpu_buffer_rsrc_t null_rsrc = make_rsrc(x, 0);
#define TERN_GEMM_DMA(BUF, XR, PR, STAGE, Q)                                                \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                 \
      (STAGE) < stages ? (dma_is_x[Q] ? (XR) : (PR)) : null_rsrc,                          \
      (lds_void_t*)(&BUF[dma_lds[Q]]), 16, dma_voff[Q],                                    \
      ((STAGE) < stages ? (STAGE) : 0) * (dma_is_x[Q] ? 128 : C::kPRow), 0, 0);
#define TERN_GEMM_ISSUE(BUF, XR, PR, STAGE) \
  _Pragma("unroll") for (int q = 0; q < C::kLoads; ++q) TERN_GEMM_DMA(BUF, XR, PR, STAGE, q)

  // MFMA operand reads.  Block b of a step covers, for the lanes of k-group
  // g, k = 16 g + 8 b .. 16 g + 8 b + 7 of the step: X chunk 2 g + b of row
  // (wm*kWM + 16 i + l16), and codes 8 b .. 8 b + 7 of 32-bit word g of
  // weight row (wn*kWN + 16 j + l16).  A8: k = 32 g + 16 b .. 32 g + 16 b +
  // 15: the same X chunk (16 int8 values) and all 16 codes of word 2 g + b.
  const uint32_t x_row0 = static_cast<uint32_t>(wm * C::kWM + l16);
  const uint32_t xo0 = x_row0 * 128u + ((static_cast<uint32_t>(2 * g + 0) ^ xswz(x_row0)) << 4);
  const uint32_t xo1 = x_row0 * 128u + ((static_cast<uint32_t>(2 * g + 1) ^ xswz(x_row0)) << 4);
  const uint32_t po = C::kXBytes + static_cast<uint32_t>(wn * C::kWN + l16) * C::kPRow +
                      (A8 ? 8u : 4u) * g;
  static_assert(C::kWM % 16 == 0, "xswz(row + 16 i) == xswz(row)");

  // (A8: the int32 sums live in the same accumulator registers, as bits.)
  using PwT = std::conditional_t<A8, u32x2_t, uint32_t>;
  f32x4_t acc[kTN][kTM];
  PwT pw[kTN];
  uint32_t tq[kTN][4];
  u32x4_t wa[kTN], wb[kTN];
  u32x4_t xa[kTM], xb[kTM];

  // Operand reads out of ring stage BUF: the 32-bit code words of every
  // weight tile (READ_PW), the X chunks of k-block 0 (READ_XA) and of k-block
  // 1 (READ_XB); READ_A is all of a step's words and k-block 0 chunks.
#define TERN_GEMM_READ_PW(BUF, J) \
  pw[J] = *reinterpret_cast<const PwT*>(&BUF[po + (J) * (16 * C::kPRow)]);
#define TERN_GEMM_READ_XA(BUF, I) xa[I] = *reinterpret_cast<const u32x4_t*>(&BUF[xo0 + (I) * 2048]);
#define TERN_GEMM_READ_XB(BUF, I) xb[I] = *reinterpret_cast<const u32x4_t*>(&BUF[xo1 + (I) * 2048]);
#define TERN_GEMM_READ_A(BUF)                                         \
  _Pragma("unroll") for (int j = 0; j < kTN; ++j) TERN_GEMM_READ_PW(BUF, j) \
  _Pragma("unroll") for (int i = 0; i < kTM; ++i) TERN_GEMM_READ_XA(BUF, i)

  // ZERO starts a new sum (the MFMA's C operand is the constant 0), so the
  // accumulators of consecutive tiles never meet in one register value.
  using kAcc = std::false_type;
  using kZero = std::true_type;
  // Before the accumulators are read: an MFMA result may be read by other
  // instructions only after up to 19 wait states.  The empty asm statements
  // order every read of acc after the s_nop block.
  auto acc_ready = [&]() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int i = 0; i < kTM; ++i) asm volatile("" : "+a"(acc[j][i]));
  };

  // Decode of weight word j (16 codes, code c in bits 2c..2c+1) in units of
  // at most two VALU instructions, so that it can be spread between MFMAs.
  // The lo units build four byte-lane vectors, tq[j][r] = (pw << (6 - 2r)) &
  // 0xC0C0C0C0: byte b of tq[j][r] holds code 4b + r in bits 6..7 and zeros
  // below, which is the high byte of the bf16 value 0 / +2 / -2 of that code.
  // A byte permute then places two such bytes over zero low bytes, giving the
  // two bf16 values of one operand register: register q of k-block h takes
  // codes 8h + 2q and 8h + 2q + 1.  Lo units 0..3 build tq[j], 4..5 the
  // k-block 0 operand wa[j] (codes 0..7); the hi units build wb[j] (codes
  // 8..15) out of the same tq[j] in the next half step.
  //
  // A8: the words are in the field-transposed packing (field 4 i + j holds
  // code 4 j + i), so (w << (6 - 2r)) & 0xC0C0C0C0 is operand register r
  // itself: byte b holds code 4 r + b as the int8 value 0 / +64 / -64.  Lo
  // unit r builds register r of wa[j] out of the first word, hi unit r
  // register r of wb[j] out of the second.
  constexpr int kLoUnits = A8 ? 4 : 6;
  constexpr int kHiUnits = A8 ? 4 : 2;
  auto lo_unit = [&](int j, int u) {
    constexpr uint32_t kTop2 = 0xC0C0C0C0u;
    if constexpr (A8) {
      wa[j][u] = (pw[j][0] << (6 - 2 * u)) & kTop2;
    } else if (u < 4) {
      tq[j][u] = (pw[j] << (6 - 2 * u)) & kTop2;
    } else {
      const uint32_t sel = u == 4 ? 0x040C000Cu : 0x050C010Cu;
      wa[j][2 * (u - 4)] = __builtin_amdgcn_perm(tq[j][1], tq[j][0], sel);
      wa[j][2 * (u - 4) + 1] = __builtin_amdgcn_perm(tq[j][3], tq[j][2], sel);
    }
  };
  auto hi_unit = [&](int j, int u) {
    if constexpr (A8) {
      wb[j][u] = (pw[j][1] << (6 - 2 * u)) & 0xC0C0C0C0u;
    } else {
      const uint32_t sel = u == 0 ? 0x060C020Cu : 0x070C030Cu;
      wb[j][2 * u] = __builtin_amdgcn_perm(tq[j][1], tq[j][0], sel);
      wb[j][2 * u + 1] = __builtin_amdgcn_perm(tq[j][3], tq[j][2], sel);
    }
  };
  auto decode_lo_all = [&]() {  // the first step's wa
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int u = 0; u < kLoUnits; ++u) lo_unit(j, u);
  };
  constexpr int kSlots = kTN * kTM;         // MFMAs per half step
  constexpr int kUnitsA = kHiUnits * kTN;   // decode units of half A
  constexpr int kUnitsB = kLoUnits * kTN;   // ... of half B
  // Half A: one X read (kTM) and kUpsA decode units per slot.  Half B: the
  // memory operations, and the decode of the next wa as late as possible.
  // Wave tiles with at least 32 MFMAs per half step start that decode once
  // the first weight words have had a few MFMAs to arrive and fit every unit
  // into the MFMA slots (several per slot when there are more units than
  // slots); smaller ones decode after all of half B's memory operations, one
  // unit per slot, and the slots past kSlots carry no MFMA.
  constexpr bool kWide = kSlots >= 32;
  constexpr int kUpsA = (kWide && kUnitsA > kSlots) ? (kUnitsA + kSlots - 1) / kSlots : 1;
  constexpr int kUpsB = (kWide && kUnitsB > kSlots) ? (kUnitsB + kSlots - 1) / kSlots : 1;
  constexpr int kUnitSlotsA = (kUnitsA + kUpsA - 1) / kUpsA;
  constexpr int kUnitSlotsB = (kUnitsB + kUpsB - 1) / kUpsB;
  constexpr int kSlotsA = kSlots > kUnitSlotsA ? kSlots : kUnitSlotsA;
  constexpr int kOpsB = kTN + C::kLoads + kTM;
  constexpr int kDecodeEarliest = kWide ? (kTN < 6 ? kTN : 6) : kOpsB;
  constexpr int kDecodeFrom =
      (kSlots - kUnitSlotsB) > kDecodeEarliest ? kSlots - kUnitSlotsB : kDecodeEarliest;
  constexpr int kSlotsB =
      kSlots > kDecodeFrom + kUnitSlotsB ? kSlots : kDecodeFrom + kUnitSlotsB;
  // An MFMA may read a VGPR only two wait states after a VALU instruction
  // wrote it.  In the wide schedules every operand is produced at least a
  // dozen slots before its MFMA (wa in the previous half B, wb in half A,
  // X chunks by LDS reads), so their MFMAs carry no padding; the small
  // schedules can put a decode unit right before the MFMA that reads its
  // result, and pad every MFMA with s_nop 1.  A CPU test checks the compiled
  // kernels for this hazard.
  constexpr bool kPad = !kWide;

  // One step out of ring stage CUR.  On entry the weight words pw, their
  // k-block 0 operands wa (and w2) and the X chunks xa of this step are in
  // registers.  Half A runs k-block 0; between its MFMAs it reads the X
  // chunks xb of k-block 1 and decodes the k-block 1 operands wb.  Then, once
  // every wave is past the barrier (the next step's stage has landed
  // everywhere and the previous step's stage is no longer read by anyone),
  // half B runs k-block 1; between its MFMAs it reads the next step's weight
  // words out of NXT, requests the step under the issue cursor into the
  // previous step's buffer DMA, reads the next step's xa, and decodes the
  // next step's wa.  The MFMAs are volatile asm and every slot ends in a
  // scheduling barrier, so this interleave is the issue order.  At every
  // barrier of the unrolled loop exactly kRing-2 steps are in flight.
#define TERN_GEMM_HALF_A(CUR, ZERO)                                                     \
  _Pragma("unroll") for (int t = 0; t < kSlotsA; ++t) {                                 \
    if (t < kSlots)                                                                     \
      mfma_op<A8, ZERO::value, kPad>(acc[t / kTM][t % kTM], wa[t / kTM], xa[t % kTM]);  \
    if (t < kTM) TERN_GEMM_READ_XB(CUR, t)                                              \
    _Pragma("unroll") for (int u = t * kUpsA; u < (t + 1) * kUpsA && u < kUnitsA; ++u)  \
      hi_unit(u / kHiUnits, u % kHiUnits);                                              \
    __builtin_amdgcn_sched_barrier(0);                                                  \
  }
#define TERN_GEMM_STEP(CUR, NXT, DMA, XR, PR, STAGE, ZERO)                                \
  {                                                                                      \
    TERN_GEMM_HALF_A(CUR, ZERO)                                                          \
    wait_vmcnt<(kRing - 3) * C::kLoads, true>();                                         \
    lds_barrier();                                                                       \
    _Pragma("unroll") for (int t = 0; t < kSlotsB; ++t) {                                \
      if (t < kSlots)                                                                    \
        mfma_op<A8, false, kPad>(acc[t / kTM][t % kTM], wb[t / kTM], xb[t % kTM]);       \
      if (t < kTN) {                                                                     \
        TERN_GEMM_READ_PW(NXT, t)                                                        \
      } else if (t < kTN + C::kLoads) {                                                  \
        TERN_GEMM_DMA(DMA, XR, PR, STAGE, t - kTN)                                       \
      } else if (t < kOpsB) {                                                            \
        TERN_GEMM_READ_XA(NXT, t - kTN - C::kLoads)                                      \
      }                                                                                  \
      if (t >= kDecodeFrom) {                                                            \
        _Pragma("unroll") for (int u = (t - kDecodeFrom) * kUpsB;                        \
                               u < (t - kDecodeFrom + 1) * kUpsB && u < kUnitsB; ++u)    \
          lo_unit(u / kLoUnits, u % kLoUnits);                                           \
      }                                                                                  \
      __builtin_amdgcn_sched_barrier(0);                                                 \
    }                                                                                    \
  }
  // Epilogue of tile t.  For MFMA tile (j, i) the lane holds output channels
  // n = wn*kWN + 16 j + 4 g + e (e = 0..3) of token m = wm*kWM + 16 i + l16.
  // The decode produced 2 T, so y = bf16(fp32(acc * s) * 0.5), which equals
  // bf16(fp32(acc / 2 * s)) exactly.  A8: the decode produced 64 T and the
  // sum is an int32, so y = bf16(fp32(fp32(acc) * fp32(s / 64)) * xs[m]).
  //
  // Whole tiles with a 16-byte aligned Y and scale vector go through LDS:
  // each wave writes 16 of its rows at a time, kEpiJ MFMA tiles (16 kEpiJ
  // columns) per pass, into its own part of the ring's last stage (lds5, or
  // lds3 in a four-stage ring; pitch kEpiPitch
  // bytes, conflict-free for the 8-byte writes) and stores them back as
  // 16-byte pieces of whole row segments (32 kEpiJ bytes per row), so that a
  // store instruction writes a few long contiguous runs instead of 16
  // scattered 32-byte ones.  kEpiJ is the largest divisor of kTN whose four
  // staging areas fit one ring stage.  That stage holds no live data here: it held
  // the tile's last stage (all reads of it end at the barrier below) and the
  // next request into it follows the next step's barrier.  Other tiles take
  // the direct path, with 8-byte stores where Y allows them.
  constexpr int kEpiJ = [] {
    int best = 0;
    for (int d = 1; d <= kTN; ++d)
      if (kTN % d == 0 && kThreads / 64 * 16 * (32 * d + 16) <= C::kStage) best = d;
    return best;
  }();
  constexpr bool kEpiLds = kEpiJ > 0;
  // The decode's factor (2 or 64), removed exactly, and the accumulator as
  // fp32 (A8: the int32 sum converted, exact below 2^24).
  constexpr float kDecode = A8 ? 0.015625f : 0.5f;
  auto acc_value = [](const f32x4_t& a) -> f32x4_t {
    if constexpr (A8)
      return __builtin_convertvector(__builtin_bit_cast(i32x4_t, a), f32x4_t);
    else
      return a;
  };
  static_assert(kEpiLds || !PERSIST, "the persistent kernel stores through LDS");
  auto epilogue = [&](int t) {
    acc_ready();
    int m0, n0;
    tile_coords(t, m0, n0);
    if (kEpiLds && (PERSIST || ((y_flags & 2) && m0 + BM <= m && n0 + BN <= n))) {
      constexpr int kEpiPitch = 32 * kEpiJ + 16;
      constexpr int kChunksPerRow = 2 * kEpiJ;                    // 16-byte pieces of a row
      constexpr int kChunks = 16 * kChunksPerRow;                 // per pass
      constexpr int kStores = (kChunks + 63) / 64;                // per lane per pass
      const uint32_t area = static_cast<uint32_t>(wave) * (16 * kEpiPitch);
      const int col0 = n0 + wn * C::kWN;
      // The factor 1/2 of the decode goes into the scale: (acc * (s / 2))
      // rounds like (acc * s) / 2 except where a result is subnormal.
      f32x4_t sc[kTN];
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        sc[j] = s != nullptr ? *reinterpret_cast<const f32x4_t*>(s + col0 + 16 * j + 4 * g) * kDecode
                             : f32x4_t{kDecode, kDecode, kDecode, kDecode};
      // A8: the scale of each of the lane's tokens (the tile is whole).
      float xsv[A8 ? kTM : 1];
      if constexpr (A8) {
#pragma unroll
        for (int i = 0; i < kTM; ++i) xsv[i] = xs[m0 + wm * C::kWM + 16 * i + l16];
      }
      const bool act_all = col0 >= act_from;
      const bool act_none = col0 + C::kWN <= act_from;
      f32x4_t bsv[EPI ? kTN : 1];
      if constexpr (EPI) {
#pragma unroll
        for (int j = 0; j < kTN; ++j)
          bsv[j] = bias != nullptr
                       ? *reinterpret_cast<const f32x4_t*>(bias + col0 + 16 * j + 4 * g)
                       : f32x4_t{};
      }
      uint32_t rd_off[kStores], st_off[kStores];
#pragma unroll
      for (int q = 0; q < kStores; ++q) {
        const int c = lane + 64 * q;
        const int row = c / kChunksPerRow;
        const int cc = c - row * kChunksPerRow;
        rd_off[q] = area + static_cast<uint32_t>(row * kEpiPitch + cc * 16);
        st_off[q] = static_cast<uint32_t>(row * ldy + cc * 8);   // 16 * ldy < 2^31 (host)
      }
      const uint32_t wr_off = area + static_cast<uint32_t>(l16 * kEpiPitch + 8 * g);
      uint16_t* const yt = y + static_cast<int64_t>(m0 + wm * C::kWM) * ldy + col0;
      // Pass p covers MFMA row block i = p / kJPasses and tiles jp .. jp +
      // kEpiJ - 1 (jp = kEpiJ (p % kJPasses)).  The passes are software
      // pipelined: pass p's staging writes and read-backs are issued, then
      // pass p + 1's accumulators are scaled and converted while those LDS
      // accesses complete, then pass p's rows are stored.  (LDS accesses of
      // one wave complete in order: the read-backs see the writes before
      // them, and the next pass's writes follow them.)
      constexpr int kJPasses = kTN / kEpiJ;
      constexpr int kPasses = kTM * kJPasses;
      u32x2_t o[2][kEpiJ];
      auto convert = [&](int p, u32x2_t (&out)[kEpiJ]) {
        const int i = p / kJPasses;
        const int jp = (p % kJPasses) * kEpiJ;
        // All of the pass's accumulator reads first, then the products, then
        // the conversions: independent instructions back to back instead of
        // dependent chains.  (The empty asm statements keep the reads here
        // instead of hoisted into one burst that needs 216 VGPRs.)
        f32x4_t v[kEpiJ];
#pragma unroll
        for (int jj = 0; jj < kEpiJ; ++jj) {
          asm volatile("" : "+a"(acc[jp + jj][i]));
          v[jj] = acc_value(acc[jp + jj][i]);
        }
#pragma unroll
        for (int jj = 0; jj < kEpiJ; ++jj) v[jj] *= sc[jp + jj];
        if constexpr (A8) {
#pragma unroll
          for (int jj = 0; jj < kEpiJ; ++jj) v[jj] *= xsv[i];
        }
        if constexpr (EPI) {
#pragma unroll
          for (int jj = 0; jj < kEpiJ; ++jj) v[jj] += bsv[jp + jj];
          // The activated columns start at act_from: all of the wave's
          // columns, none of them (no GELU), or a boundary inside them.
          if (act_all) {
#pragma unroll
            for (int jj = 0; jj < kEpiJ; ++jj)
#pragma unroll
              for (int e = 0; e < 4; ++e) v[jj][e] = gelu_tanh_f32(v[jj][e]);
          } else if (!act_none) {
#pragma unroll
            for (int jj = 0; jj < kEpiJ; ++jj) {
              const int c0 = col0 + 16 * (jp + jj) + 4 * g;
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (c0 + e >= act_from) v[jj][e] = gelu_tanh_f32(v[jj][e]);
            }
          }
        }
#pragma unroll
        for (int jj = 0; jj < kEpiJ; ++jj) {
          out[jj][0] = pack_bf16x2(v[jj][0], v[jj][1]);
          out[jj][1] = pack_bf16x2(v[jj][2], v[jj][3]);
        }
      };
      convert(0, o[0]);
      lds_barrier();
#pragma unroll
      for (int p = 0; p < kPasses; ++p) {
#pragma unroll
        for (int jj = 0; jj < kEpiJ; ++jj)
          if constexpr (RING == 6)
            *reinterpret_cast<u32x2_t*>(&lds5[wr_off + 32 * jj]) = o[p % 2][jj];
          else
            *reinterpret_cast<u32x2_t*>(&lds3[wr_off + 32 * jj]) = o[p % 2][jj];
        u32x4_t v[kStores];
#pragma unroll
        for (int q = 0; q < kStores; ++q)
          if (kChunks % 64 == 0 || lane + 64 * q < kChunks)
            v[q] = RING == 6 ? *reinterpret_cast<const u32x4_t*>(&lds5[rd_off[q]])
                             : *reinterpret_cast<const u32x4_t*>(&lds3[rd_off[q]]);
        if (p + 1 < kPasses) convert(p + 1, o[(p + 1) % 2]);
        uint16_t* const yi =
            yt + static_cast<int64_t>(16 * (p / kJPasses)) * ldy + 16 * kEpiJ * (p % kJPasses);
#pragma unroll
        for (int q = 0; q < kStores; ++q)
          if (kChunks % 64 == 0 || lane + 64 * q < kChunks)
            *reinterpret_cast<u32x4_t*>(yi + st_off[q]) = v[q];
      }
      return;
    }
    if constexpr (!PERSIST) {
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        const int ng = n0 + wn * C::kWN + 16 * j + 4 * g;
        float sc[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[e] = (ng + e < n) ? (s != nullptr ? s[ng + e] : 1.0f) : 0.0f;
        if constexpr (A8) {
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[e] *= kDecode;
        }
        float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (EPI) {
#pragma unroll
          for (int e = 0; e < 4; ++e) bv[e] = (bias != nullptr && ng + e < n) ? bias[ng + e] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
          const int mg = m0 + wm * C::kWM + 16 * i + l16;
          const f32x4_t av = acc_value(acc[j][i]);
          float xsm = 0.0f;
          if constexpr (A8) xsm = mg < m ? xs[mg] : 0.0f;
          __bf16 b[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float z = A8 ? (av[e] * sc[e]) * xsm : (av[e] * sc[e]) * 0.5f;
            if constexpr (EPI) {
              z += bv[e];
              if (ng + e >= act_from) z = gelu_tanh_f32(z);
            }
            b[e] = static_cast<__bf16>(z);
          }
          if (mg >= m) continue;
          uint16_t* yr = y + static_cast<int64_t>(mg) * ldy + ng;
          if ((y_flags & 1) && ng + 4 <= n) {
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
    }
  };

  // One unrolled iteration: steps st .. st + kRing - 1 out of ring stages 0 ..
  // kRing - 1.  The first request is stage st + kRing - 1 of this tile, the
  // others stages B0 .. B0 + kRing - 2 of the tile with resources BX, BP.
#define TERN_GEMM_ITER6(BX, BP, B0, ZERO)                                         \
  /* several statements: use inside braces */                                     \
  TERN_GEMM_STEP(lds0, lds1, lds5, cur_xr, cur_pr, st + kRing - 1, ZERO)          \
  TERN_GEMM_STEP(lds1, lds2, lds0, BX, BP, (B0), kAcc)                            \
  TERN_GEMM_STEP(lds2, lds3, lds1, BX, BP, (B0) + 1, kAcc)                        \
  TERN_GEMM_STEP(lds3, lds4, lds2, BX, BP, (B0) + 2, kAcc)                        \
  TERN_GEMM_STEP(lds4, lds5, lds3, BX, BP, (B0) + 3, kAcc)                        \
  TERN_GEMM_STEP(lds5, lds0, lds4, BX, BP, (B0) + 4, kAcc)
#define TERN_GEMM_ITER4(BX, BP, B0, ZERO)                                         \
  TERN_GEMM_STEP(lds0, lds1, lds3, cur_xr, cur_pr, st + kRing - 1, ZERO)          \
  TERN_GEMM_STEP(lds1, lds2, lds0, BX, BP, (B0), kAcc)                            \
  TERN_GEMM_STEP(lds2, lds3, lds1, BX, BP, (B0) + 1, kAcc)                        \
  TERN_GEMM_STEP(lds3, lds0, lds2, BX, BP, (B0) + 2, kAcc)
#define TERN_GEMM_ITER(BX, BP, B0, ZERO)                                          \
  if constexpr (RING == 6) {                                                      \
    TERN_GEMM_ITER6(BX, BP, B0, ZERO)                                             \
  } else {                                                                        \
    TERN_GEMM_ITER4(BX, BP, B0, ZERO)                                             \
  }

  __amdgpu_buffer_rsrc_t cur_xr, cur_pr;
  tile_rsrc(0, cur_xr, cur_pr);
  TERN_GEMM_ISSUE(lds0, cur_xr, cur_pr, 0)
  TERN_GEMM_ISSUE(lds1, cur_xr, cur_pr, 1)
  TERN_GEMM_ISSUE(lds2, cur_xr, cur_pr, 2)
  if constexpr (RING == 6) {
    TERN_GEMM_ISSUE(lds3, cur_xr, cur_pr, 3)
    TERN_GEMM_ISSUE(lds4, cur_xr, cur_pr, 4)
  }
  wait_vmcnt<(kRing - 2) * C::kLoads, true>();
  lds_barrier();
  TERN_GEMM_READ_A(lds0)
  decode_lo_all();
  // The first MFMA reads wa right after this decode: two wait states (the
  // schedule of the loop keeps every other decode far from its MFMA).
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 1");
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (PERSIST) {
    for (int t = 0; t < my_tiles; ++t) {
      // In the tile's last iteration the requests after the first continue
      // with stages 0 .. kRing - 2 of the next tile, or, after the last tile,
      // with dummy re-loads of this tile's last stage.
#define TERN_GEMM_PITER(ZERO)                               \
      {                                                     \
        __amdgpu_buffer_rsrc_t bx = cur_xr, bp = cur_pr;    \
        int b0 = st + kRing;                                \
        if (st + kRing == stages) {                         \
          if (t + 1 < my_tiles) {                           \
            tile_rsrc(t + 1, bx, bp);                       \
            b0 = 0;                                         \
          } else {                                          \
            b0 = stages;                                    \
          }                                                 \
        }                                                   \
        TERN_GEMM_ITER(bx, bp, b0, ZERO)                    \
      }
      int st = 0;
      TERN_GEMM_PITER(kZero)
      for (st = kRing; st < stages; st += kRing) TERN_GEMM_PITER(kAcc)
#undef TERN_GEMM_PITER
      epilogue(t);
      if (t + 1 < my_tiles) tile_rsrc(t + 1, cur_xr, cur_pr);
    }
    wait_vmcnt<0>();  // no DMA may outlive the workgroup's LDS
  } else {
    // One tile; the last iteration may run past the end of K on zeros.
    int st = 0;
    TERN_GEMM_ITER(cur_xr, cur_pr, st + kRing, kZero)
    for (st = kRing; st < stages; st += kRing) {
      TERN_GEMM_ITER(cur_xr, cur_pr, st + kRing, kAcc)
    }
    wait_vmcnt<0>();  // no DMA may outlive the workgroup's LDS
    epilogue(0);
  }
#undef TERN_GEMM_ITER
#undef TERN_GEMM_ITER6
#undef TERN_GEMM_ITER4
#undef TERN_GEMM_STEP
#undef TERN_GEMM_HALF_A
#undef TERN_GEMM_ISSUE
#undef TERN_GEMM_DMA
#undef TERN_GEMM_READ_A
#undef TERN_GEMM_READ_PW
#undef TERN_GEMM_READ_XA
#undef TERN_GEMM_READ_XB
#endif  // __HIP_DEVICE_COMPILE__
}

// k == 0: the sum is empty, so Y = bf16(f(0 * s + b)): zero, or the
// epilogue applied to the bias alone.
__global__ void fill_empty_sum(uint16_t* y, int m, int n, int ldy, const float* bias,
                               int act_from) {
  const int64_t total = static_cast<int64_t>(m) * n;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = i / n;
    const int c = static_cast<int>(i - r * n);
    float z = bias != nullptr ? bias[c] : 0.0f;
    if (c >= act_from) z = gelu_tanh_f32(z);
    y[r * ldy + c] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(z));
  }
}

// Workgroups per launch: persistent (a multiple of 8, at most one per CU)
// when the K steps can run as one ring stream across tiles, else one per
// tile.
constexpr int kPersistentGrid = 256;
constexpr int64_t kSmallMaxM = 32;

template <int BM, int BN, int WAVES_M, int GM, int WPE, bool EPI, bool A8 = false, int RING = 6>
hipError_t launch_tiles(const void* x, int64_t m, int64_t k, int64_t ldx, const float* xs,
                        const uint8_t* p, int64_t n, int64_t ldp, const float* s,
                        const float* bias, int act_from, uint16_t* y, int64_t ldy,
                        hipStream_t stream) {
  const int tiles_m = static_cast<int>((m + BM - 1) / BM);
  const int tiles_n = static_cast<int>((n + BN - 1) / BN);
  const int64_t tiles = static_cast<int64_t>(tiles_m) * tiles_n;
  const int stages = static_cast<int>(k / TileCfg<BM, BN, WAVES_M, A8>::kBK);
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  // Bit 0: 8-byte stores of Y; bit 1: 16-byte stores of Y, 16-byte loads of
  // the scales (and of the bias) and 32-bit offsets within 16 rows of Y.
  const int y_flags =
      (((reinterpret_cast<uintptr_t>(y) & 7) == 0 && ldy % 4 == 0) ? 1 : 0) |
      (((reinterpret_cast<uintptr_t>(y) & 15) == 0 && ldy % 8 == 0 && ldy < (int64_t{1} << 27) &&
        (reinterpret_cast<uintptr_t>(s) & 15) == 0 &&
        (reinterpret_cast<uintptr_t>(bias) & 15) == 0) ? 2 : 0);
  // The persistent kernel takes whole tiles only (its epilogue has no edge
  // handling) and needs the ring stream to restart at a tile boundary.
  if constexpr (WPE == 1) {
    if (stages % RING == 0 && tiles > kPersistentGrid && m % BM == 0 && n % BN == 0 &&
        (y_flags & 2)) {
      hipLaunchKernelGGL((gemm_ternary_mfma<BM, BN, WAVES_M, GM, true, WPE, EPI, A8, RING>),
                         dim3(kPersistentGrid), dim3(kThreads), 0, stream, xb,
                         static_cast<int>(m), static_cast<int>(k), static_cast<int>(ldx), xs, p,
                         static_cast<int>(n), static_cast<int>(ldp), s, bias, act_from, y,
                         static_cast<int>(ldy), tiles_m, tiles_n, y_flags);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_ternary_mfma<BM, BN, WAVES_M, GM, false, WPE, EPI, A8, RING>),
                     dim3(static_cast<unsigned>(tiles)), dim3(kThreads), 0, stream, xb,
                     static_cast<int>(m), static_cast<int>(k), static_cast<int>(ldx), xs, p,
                     static_cast<int>(n), static_cast<int>(ldp), s, bias, act_from, y,
                     static_cast<int>(ldy), tiles_m, tiles_n, y_flags);
  return hipGetLastError();
}

template <bool EPI>
hipError_t launch_big(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const uint8_t* p,
                      int64_t n, int64_t ldp, const float* s, const float* bias, int act_from,
                      uint16_t* y, int64_t ldy, hipStream_t stream) {
  // Layers with at least one 144 x 384 tile per CU use the big tile (one
  // workgroup per CU, 147 KiB of LDS).  Smaller layers that 64 x 576 tiles
  // cut into exactly one tile per CU use those (wave tile 64 x 144, still on
  // the wide schedule; e.g. M = 2048, N = 4608).  Others use 64-row tiles,
  // two workgroups per CU, with 256 or 128 output channels per tile,
  // whichever still gives two tiles per CU, so that every CU has work.
  const auto tiles = [&](int64_t bm, int64_t bn) { return ((m + bm - 1) / bm) * ((n + bn - 1) / bn); };
  if (tiles(144, 384) >= kPersistentGrid)
    return launch_tiles<144, 384, 1, 4, 1, EPI>(x, m, k, ldx, nullptr, p, n, ldp, s, bias,
                                                act_from, y, ldy, stream);
  if (m % 64 == 0 && n % 576 == 0 && tiles(64, 576) == kPersistentGrid)
    return launch_tiles<64, 576, 1, 4, 1, EPI>(x, m, k, ldx, nullptr, p, n, ldp, s, bias,
                                               act_from, y, ldy, stream);
  // Layers that 64-token tiles of 96, 144 or 192 channels cut into at most
  // one tile per CU, with K of at least 2048 (the DiT MLP down-projection at
  // 2048 tokens, 64 to 256 tokens on a wide weight): the workgroup's four
  // waves split K (gemm_ksplit.hip).
  if (gemm_ksplit_fits(m, k, n))
    return launch_gemm_ksplit(x, m, k, ldx, p, n, ldp, s, bias, act_from, y, ldy, stream);
  if (tiles(64, 256) >= 2 * kPersistentGrid)
    return launch_tiles<64, 256, 1, 4, 2, EPI>(x, m, k, ldx, nullptr, p, n, ldp, s, bias,
                                               act_from, y, ldy, stream);
  return launch_tiles<64, 128, 1, 4, 2, EPI>(x, m, k, ldx, nullptr, p, n, ldp, s, bias, act_from,
                                             y, ldy, stream);
}

template <bool EPI>
hipError_t launch_big_a8(const int8_t* q, int64_t m, int64_t k, int64_t ldq, const float* xs,
                         const uint8_t* p8, int64_t n, int64_t ldp8, const float* s,
                         const float* bias, int act_from, uint16_t* y, int64_t ldy,
                         hipStream_t stream) {
  // The int8 stage holds K = 128.  Large layers use 144 x 384 tiles (the
  // bf16 kernel's wave tile, 54 MFMAs per half step) in a four-stage ring of
  // 30 KiB stages (120 KiB of LDS); two stages in flight cover the memory
  // latency, since an int8 step does as many MFMAs as a bf16 one.  Layers
  // that 64 x 576 tiles cut into exactly one tile per CU use those (six
  // stages of 26 KiB); 144 x 256 tiles with six stages take the layers with
  // fewer than 256 144 x 384 tiles but at least 256 of their own; smaller
  // layers use 64 x 128 tiles, two workgroups per CU.
  const auto tiles = [&](int64_t bm, int64_t bn) { return ((m + bm - 1) / bm) * ((n + bn - 1) / bn); };
  if (m % 64 == 0 && n % 576 == 0 && tiles(64, 576) == kPersistentGrid)
    return launch_tiles<64, 576, 1, 4, 1, EPI, true>(q, m, k, ldq, xs, p8, n, ldp8, s, bias,
                                                     act_from, y, ldy, stream);
  if (tiles(144, 384) >= kPersistentGrid)
    return launch_tiles<144, 384, 1, 4, 1, EPI, true, 4>(q, m, k, ldq, xs, p8, n, ldp8, s, bias,
                                                         act_from, y, ldy, stream);
  if (tiles(144, 256) >= kPersistentGrid)
    return launch_tiles<144, 256, 1, 4, 1, EPI, true>(q, m, k, ldq, xs, p8, n, ldp8, s, bias,
                                                      act_from, y, ldy, stream);
  return launch_tiles<64, 128, 1, 4, 2, EPI, true>(q, m, k, ldq, xs, p8, n, ldp8, s, bias,
                                                   act_from, y, ldy, stream);
}

}  // namespace

hipError_t launch_gemm(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const uint8_t* p,
                       int64_t n, int64_t ldp, const float* s, const float* bias,
                       int64_t act_from, uint16_t* y, int64_t ldy, hipStream_t stream) {
  const int af = static_cast<int>(act_from);
  if (k == 0) {
    int64_t blocks = (m * n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_empty_sum, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       y, static_cast<int>(m), static_cast<int>(n), static_cast<int>(ldy), bias,
                       af);
    return hipGetLastError();
  }
  const bool epi = bias != nullptr || act_from < n;
  // A few tokens: the weight stream dominates; see gemm_small.hip.
  if (m <= kSmallMaxM)
    return launch_gemm_small(x, m, k, ldx, p, n, ldp, s, bias, act_from, y, ldy, stream);
  if (epi) return launch_big<true>(x, m, k, ldx, p, n, ldp, s, bias, af, y, ldy, stream);
  return launch_big<false>(x, m, k, ldx, p, n, ldp, s, nullptr, af, y, ldy, stream);
}

hipError_t launch_gemm_a8(const int8_t* q, int64_t m, int64_t k, int64_t ldq, const float* xs,
                          const uint8_t* p8, int64_t n, int64_t ldp8, const float* s,
                          const float* bias, int64_t act_from, uint16_t* y, int64_t ldy,
                          hipStream_t stream) {
  const int af = static_cast<int>(act_from);
  if (k == 0) {
    int64_t blocks = (m * n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_empty_sum, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       y, static_cast<int>(m), static_cast<int>(n), static_cast<int>(ldy), bias,
                       af);
    return hipGetLastError();
  }
  // A few tokens: the weight stream dominates; see gemm_small.hip.
  if (m <= kSmallMaxM)
    return launch_gemm_small_a8(q, m, k, ldq, xs, p8, n, ldp8, s, bias, act_from, y, ldy, stream);
  if (bias != nullptr || act_from < n)
    return launch_big_a8<true>(q, m, k, ldq, xs, p8, n, ldp8, s, bias, af, y, ldy, stream);
  return launch_big_a8<false>(q, m, k, ldq, xs, p8, n, ldp8, s, nullptr, af, y, ldy, stream);
}

}  // namespace tern
