// Ternary linear layer for layers with few output tiles and a long K:
//   Y = bf16(f((X . T^T) (.) s + b)), bf16 X, 2-bit packed T.
//
// "1.58-bit FLUX" (arXiv 2412.18653) builds a linear kernel for 1.58-bit
// weights with unquantized activations (section 1 contributions, section
// 3.2, section 4 limitations), and "TerDiT: Ternary Diffusion Models with
// Transformers" (abstract) applies the same weights to DiT-style models.  A
// DiT MLP down-projection at 2048 tokens (X [2048, 4608], output 1152
// channels) has only 256 output tiles of 64 x 144 but 4608 terms per sum, and
// a layer of 64 to 256 tokens on a wide weight (the single-stream
// in-projection's 21504 x 3072) few tiles of any size: one workgroup per tile
// with the whole K in sequence leaves the matrix cores waiting on a long
// dependent stream, and smaller tiles re-read X many times.
//
// Design:
//  * One workgroup per 64 (tokens) x 16 TN (channels) tile, TN = 6, 9 or 12
//    (the narrowest whose tiles fill the chip at most once), four waves that
//    split K: wave w takes the K steps w, w + 4, w + 8, ... (64 values of K
//    per step).  Each wave owns the whole tile as TN x 4 tiles of
//    v_mfma_f32_16x16x32_bf16 (16 TN accumulator registers): a decoded weight
//    operand feeds 4 MFMAs, an X operand TN.
//  * Every wave streams its own steps through its own three-stage ring in
//    LDS by LDS-DMA buffer loads (16 bytes per lane; per step X 64 rows x 128
//    bytes and the packed weights 16 TN rows x 16 bytes, padded to a multiple
//    of 64 rows that read as zero): there is no workgroup barrier in the
//    loop, and a wave waits only for its own loads.  Each ring stage index is its own
//    LDS object (holding that stage for all four waves), so the compiler
//    tracks the DMA writes of the stages apart.
//  * The data layout in a stage, the operand reads and the decode are those
//    of gemm.hip: 16-byte X chunks XOR-swizzled by ((row >> 1) & 7), the
//    weights kept packed and decoded between the MFMAs (15 VALU instructions
//    per 16 codes, bf16 values 0 / +2 / -2, the factor 2 removed in the
//    epilogue).  The weights are the MFMA's A operand, X the B operand, so a
//    lane ends with four consecutive channels of one token.
//  * After the last step the four partial tiles meet in LDS (the rings are
//    free by then): wave v writes its sums for the token blocks other than
//    v, and wave w adds, for token block w, the partials in wave order 0, 1,
//    2, 3, a fixed order (repeated calls give identical bits).  It then
//    applies the scale (and the bias and GELU), rounds once to bf16 and
//    stores its 16 token rows.
//  * Workgroups are renumbered so that each XCD (one L2 each) takes a
//    contiguous range of tiles, in token-major order (the channel tiles of a
//    64-token block run on one XCD and share its X rows in that L2) or, where
//    that fetches fewer bytes (the weights outweigh X: a few token blocks on a
//    wide weight), channel-major (the token blocks of a channel tile share
//    its weight rows).
#include <type_traits>

#include "gemm_common.h"
#include "internal.h"

namespace tern {
namespace {

constexpr int kKsThreads = 256;  // four waves
constexpr int kKsTM = 4;         // 16-token blocks per tile: one per wave in the reduction
constexpr int kKsRing = 3;       // stages per wave ring

// s_waitcnt: this wave's vector-memory counter <= N (LDS counter untouched).
template <int N>
__device__ inline void ks_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Slot of the logical 16-byte X chunk c of LDS row r: c ^ ks_xswz(r).  The 16
// rows that one 16-lane group of an operand read touches (one logical chunk)
// land in 16 distinct 16-byte bank groups.
__device__ inline uint32_t ks_xswz(uint32_t r) { return (r >> 1) & 7u; }

template <int TN>
struct KsCfg {
  static constexpr int kBM = 16 * kKsTM;            // tokens per tile
  static constexpr int kBN = 16 * TN;               // channels per tile
  static constexpr int kXBytes = kBM * 128;         // X of one step: 64 bf16 per row
  static constexpr int kXInstr = kXBytes / 1024;    // DMA instructions of 8 rows
  static constexpr int kPInstr = (kBN + 63) / 64;   // DMA instructions of 64 weight rows
  // Weight bytes of a stage: the DMA rows, and at least TN - 8 KiB, so that a
  // wave's three stages hold its 3 TN partial tiles of 1 KiB in the hand-over.
  static constexpr int kPBytes = (kPInstr > TN - 8 ? kPInstr : TN - 8) * 1024;
  static constexpr int kStage = kXBytes + kPBytes;  // one wave's stage
  static constexpr int kLoads = kXInstr + kPInstr;  // DMA instructions per step
  static constexpr int kSlots = TN * kKsTM;         // MFMAs per half step
  static constexpr int kPerArr = kStage / 1024;     // 1 KiB partial tiles per stage object
  // Where the next step's decode runs: the tq vectors of words 0 .. kTqA - 1
  // in half A from slot kTqA0 on, those of the other words at the start of
  // half B, then the wa operands of every word from slot kWaB0 of half B.
  static constexpr int kTqA = TN == 6 ? 4 : (TN == 9 ? 5 : 8);
  static constexpr int kTqA0 = TN == 6 ? 8 : 16;
  static constexpr int kWaB0 = 4 * (TN - kTqA);
  static_assert(3 * TN <= kKsRing * kPerArr, "a wave's partial tiles fit in its ring");
  static_assert(kLoads + TN + kKsTM <= kSlots, "half B has a slot for every memory operation");
  static_assert(4 * kKsRing * kStage <= 160 * 1024, "LDS");
};

// Maps the hardware workgroup id to a logical tile: workgroups are dealt to
// the 8 XCDs round-robin, and renumbering gives each XCD a contiguous range.
__device__ inline int ks_logical_tile(int bid, int grid) {
  const int xcd = bid & 7;
  const int local = bid >> 3;
  const int per = grid >> 3;
  const int rem = grid & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

__device__ inline uint32_t ks_pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// y_flags bit 0: Y rows allow 8-byte stores (y 8-byte aligned, ldy % 4 == 0);
// bit 1: the logical tiles run in channel-major order (tile t covers channel
// tile t / tiles_m and token block t % tiles_m) instead of token-major.
template <int TN, bool EPI>
__global__ __launch_bounds__(kKsThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_ternary_ksplit(const uint8_t* __restrict__ x, int m, int k, int ldx,
                         const uint8_t* __restrict__ p, int n, int ldp,
                         const float* __restrict__ s, const float* __restrict__ bias,
                         int act_from, uint16_t* __restrict__ y, int ldy, int tiles_n,
                         int y_flags) {
#if defined(__HIP_DEVICE_COMPILE__)
  // (The body uses LDS address-space casts that only the device pass accepts.)
  using C = KsCfg<TN>;
  constexpr int TM = kKsTM;
  __shared__ __attribute__((aligned(1024))) uint8_t ks0[4 * C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t ks1[4 * C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t ks2[4 * C::kStage];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  __builtin_assume(wave >= 0 && wave < 4);
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const uint32_t wbase = static_cast<uint32_t>(wave) * C::kStage;

  const int logical = ks_logical_tile(blockIdx.x, gridDim.x);
  const int tiles_m = (m + C::kBM - 1) / C::kBM;
  int tm, tn;
  if (y_flags & 2) {
    tn = logical / tiles_m;
    tm = logical - tn * tiles_m;
  } else {
    tm = logical / tiles_n;
    tn = logical - tm * tiles_n;
  }
  const int m0 = tm * C::kBM;
  const int n0 = tn * C::kBN;
  const int rows_m = (m - m0) < C::kBM ? (m - m0) : C::kBM;
  const int rows_n = (n - n0) < C::kBN ? (n - n0) : C::kBN;
  const int ldxb = ldx * 2;  // X pitch in bytes (< 2^24, checked by the host)

  // Buffer resources rebased at the tile's first row: rows past the last
  // valid one read as zero; a step past this wave's last is requested
  // through an empty resource and arrives as zeros.
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(x + static_cast<int64_t>(m0) * ldxb,
                static_cast<uint32_t>(static_cast<int64_t>(rows_m - 1) * ldxb + 2 * static_cast<int64_t>(k)));
  const __amdgpu_buffer_rsrc_t pr =
      make_rsrc(p + static_cast<int64_t>(n0) * ldp,
                static_cast<uint32_t>(static_cast<int64_t>(rows_n - 1) * ldp + k / 4));
  const __amdgpu_buffer_rsrc_t null_rsrc = make_rsrc(x, 0);

  const int stages = k >> 6;
  const int my_steps = wave < stages ? (stages - 1 - wave) / 4 + 1 : 0;

  // DMA plan of a step.  X load q (q < kXInstr) fills stage bytes [1024 q,
  // +1024): rows 8 q + lane / 8, slot lane % 8, which holds logical chunk
  // (lane % 8) ^ ks_xswz(row).  Weight load q fills [kXBytes + 1024 q, +1024):
  // row 64 q + lane, 16 bytes.
  uint32_t voff[C::kLoads];
#pragma unroll
  for (int q = 0; q < C::kLoads; ++q) {
    if (q < C::kXInstr) {
      const uint32_t r = 8u * q + (lane >> 3);
      voff[q] = r * static_cast<uint32_t>(ldxb) + 16u * ((lane & 7) ^ ks_xswz(r));
    } else {
      voff[q] = (64u * (q - C::kXInstr) + lane) * static_cast<uint32_t>(ldp);
    }
  }
#define KS_LOFF(Q) ((Q) < C::kXInstr ? 1024 * (Q) : C::kXBytes + 1024 * ((Q) - C::kXInstr))
#define KS_DMA(BUF, ST, Q)                                                                 \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                \
      (ST) < my_steps ? ((Q) < C::kXInstr ? xr : pr) : null_rsrc,                          \
      (lds_void_t*)(&BUF[wbase + KS_LOFF(Q)]), 16, voff[Q],                                \
      ((ST) < my_steps ? wave + 4 * (ST) : 0) * ((Q) < C::kXInstr ? 128 : 16), 0, 0);
#define KS_ISSUE(BUF, ST) \
  _Pragma("unroll") for (int q = 0; q < C::kLoads; ++q) KS_DMA(BUF, ST, q)

  // Operand reads.  For the lanes of k-group g, k-block b of a step covers
  // k = 16 g + 8 b .. 16 g + 8 b + 7: X chunk 2 g + b of token row 16 i +
  // l16, and codes 8 b .. 8 b + 7 of 32-bit word g of weight row 16 j + l16.
  const uint32_t xo0 = wbase + static_cast<uint32_t>(l16) * 128u +
                       ((static_cast<uint32_t>(2 * g) ^ ks_xswz(l16)) << 4);
  const uint32_t xo1 = wbase + static_cast<uint32_t>(l16) * 128u +
                       ((static_cast<uint32_t>(2 * g + 1) ^ ks_xswz(l16)) << 4);
  const uint32_t po = wbase + C::kXBytes + static_cast<uint32_t>(l16) * 16u + 4u * g;
#define KS_READ_PW(BUF, J) pw[J] = *reinterpret_cast<const uint32_t*>(&BUF[po + (J) * 256]);
#define KS_READ_XA(BUF, I) xa[I] = *reinterpret_cast<const u32x4_t*>(&BUF[xo0 + (I) * 2048]);
#define KS_READ_XB(BUF, I) xb[I] = *reinterpret_cast<const u32x4_t*>(&BUF[xo1 + (I) * 2048]);

  f32x4_t acc[TN][TM];
  uint32_t pw[TN];
  uint32_t tq[TN][4];
  u32x4_t wa[TN], wb[TN];
  u32x4_t xa[TM], xb[TM];

  // Decode of weight word j in units of two VALU instructions.  Lo units 0..3
  // build tq[j][r] = (pw << (6 - 2r)) & 0xC0C0C0C0 (code 4 b + r in the top
  // bits of byte b: the high byte of its bf16 value 0 / +2 / -2), lo units 4
  // and 5 the k-block 0 operand wa[j] (codes 0..7) with byte permutes; the
  // two hi units build wb[j] (codes 8..15) out of the same tq[j].
  auto lo_unit = [&](int j, int u) {
    if (u < 4) {
      tq[j][u] = (pw[j] << (6 - 2 * u)) & 0xC0C0C0C0u;
    } else {
      const uint32_t sel = u == 4 ? 0x040C000Cu : 0x050C010Cu;
      wa[j][2 * (u - 4)] = __builtin_amdgcn_perm(tq[j][1], tq[j][0], sel);
      wa[j][2 * (u - 4) + 1] = __builtin_amdgcn_perm(tq[j][3], tq[j][2], sel);
    }
  };
  auto hi_unit = [&](int j, int u) {
    const uint32_t sel = u == 0 ? 0x060C020Cu : 0x070C030Cu;
    wb[j][2 * u] = __builtin_amdgcn_perm(tq[j][1], tq[j][0], sel);
    wb[j][2 * u + 1] = __builtin_amdgcn_perm(tq[j][3], tq[j][2], sel);
  };
  auto mfma = [&](f32x4_t& a, const u32x4_t& w, const u32x4_t& xv) {
    mfma16<false, false>(a, __builtin_bit_cast(bf16x8_t, w), __builtin_bit_cast(bf16x8_t, xv));
  };

  // The sums start at zero (a wave may have no step at all when K < 256).
  // The asm statements keep the writes here; the s_nop below keeps two wait
  // states between them and the first MFMA.
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      acc[j][i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      asm volatile("" : "+a"(acc[j][i]));
    }

  // Half A of a step: k-block 0 (wa x xa).  Between its MFMAs: the X chunks
  // of k-block 1 (xb) are read out of CUR; after the wait for the next step's
  // loads, its weight words are read out of NXT; the k-block 1 operands wb of
  // this step are decoded (the two hi units of each word), and the first part
  // of the next step's decode (the tq vectors of words 0 .. kTqA - 1) follows
  // each word's hi units.  Half B: k-block 1 (wb x xb).  Between its MFMAs: the step three
  // ahead is requested into CUR (every read of CUR is complete: its last ones,
  // the xb chunks, feed the first MFMAs of this half), the next step's
  // k-block 0 X chunks are read out of NXT, and the rest of the next step's
  // decode runs (tq of the other words, then every wa).  Each slot ends in a
  // scheduling barrier, so this interleave is the issue order, with at most
  // two decode units (four VALU instructions) per MFMA; every VALU-written
  // operand is written several slots before the MFMA that reads it.
  static_assert(TM + 2 * TN <= C::kSlots && C::kTqA0 + 4 * C::kTqA <= C::kSlots, "half A slots");
  static_assert(C::kTqA0 >= TM + 2, "a word's tq vectors follow its hi units");
  static_assert(C::kLoads + TM <= C::kSlots && C::kWaB0 + 2 * TN <= C::kSlots, "half B slots");
#define KS_STEP(CUR, NXT, ST)                                                              \
  {                                                                                       \
    _Pragma("unroll") for (int t = 0; t < C::kSlots; ++t) {                               \
      mfma(acc[t / TM][t % TM], wa[t / TM], xa[t % TM]);                                  \
      if (t < TM) {                                                                       \
        KS_READ_XB(CUR, t)                                                                \
      }                                                                                   \
      if (t == TM) ks_wait_vmcnt<C::kLoads>();                                            \
      if (t >= TM && t < TM + TN) {                                                       \
        KS_READ_PW(NXT, t - TM)                                                           \
      }                                                                                   \
      if (t >= TM && t < TM + 2 * TN) hi_unit((t - TM) / 2, (t - TM) % 2);                \
      if (t >= C::kTqA0 && t < C::kTqA0 + 4 * C::kTqA)                                    \
        lo_unit((t - C::kTqA0) / 4, (t - C::kTqA0) % 4);                                  \
      __builtin_amdgcn_sched_barrier(0);                                                  \
    }                                                                                     \
    _Pragma("unroll") for (int t = 0; t < C::kSlots; ++t) {                               \
      mfma(acc[t / TM][t % TM], wb[t / TM], xb[t % TM]);                                  \
      if (t < C::kLoads) {                                                                \
        KS_DMA(CUR, (ST) + 3, t)                                                          \
      } else if (t < C::kLoads + TM) {                                                    \
        KS_READ_XA(NXT, t - C::kLoads)                                                    \
      }                                                                                   \
      if (t < C::kWaB0) lo_unit(C::kTqA + t / 4, t % 4);                                  \
      if (t >= C::kWaB0 && t < C::kWaB0 + 2 * TN)                                         \
        lo_unit((t - C::kWaB0) / 2, 4 + (t - C::kWaB0) % 2);                              \
      __builtin_amdgcn_sched_barrier(0);                                                  \
    }                                                                                     \
  }

  // Prologue: steps 0, 1, 2 requested, step 0's operands read and decoded.
  KS_ISSUE(ks0, 0)
  KS_ISSUE(ks1, 1)
  KS_ISSUE(ks2, 2)
  ks_wait_vmcnt<2 * C::kLoads>();
#pragma unroll
  for (int j = 0; j < TN; ++j) KS_READ_PW(ks0, j)
#pragma unroll
  for (int i = 0; i < TM; ++i) KS_READ_XA(ks0, i)
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int u = 0; u < 6; ++u) lo_unit(j, u);
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 1");
  __builtin_amdgcn_sched_barrier(0);

  // Three steps per iteration, one per ring stage; steps past my_steps run on
  // zeros (the last iteration may have one or two of them).
  for (int st = 0; st < my_steps; st += 3) {
    KS_STEP(ks0, ks1, st)
    KS_STEP(ks1, ks2, st + 1)
    KS_STEP(ks2, ks0, st + 2)
  }
  ks_wait_vmcnt<0>();  // the requests past the end are in flight too

  // The channel scales (and biases) of this lane's outputs, requested now so
  // that they arrive during the hand-over below: buffer loads without a
  // branch (the range check is per 4-byte word, so channels past n read as
  // zero).  A null scale vector means unit scales (the input-gradient
  // product).
  const bool unit = s == nullptr;
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(unit ? p : reinterpret_cast<const uint8_t*>(s + n0),
                unit ? 0u : static_cast<uint32_t>(rows_n * 4));
  const __amdgpu_buffer_rsrc_t brs =
      make_rsrc(bias == nullptr ? p : reinterpret_cast<const uint8_t*>(bias + n0),
                (!EPI || bias == nullptr) ? 0u : static_cast<uint32_t>(rows_n * 4));
  f32x4_t sc[TN];
  f32x4_t bv[EPI ? TN : 1];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const uint32_t off = static_cast<uint32_t>((16 * j + 4 * g) * 4);
    sc[j] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(srs, off, 0, 0));
    if constexpr (EPI)
      bv[j] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(brs, off, 0, 0));
  }
#undef KS_STEP
#undef KS_ISSUE
#undef KS_DMA
#undef KS_LOFF
#undef KS_READ_PW
#undef KS_READ_XA
#undef KS_READ_XB

  // Every MFMA result is ready 19 wait states after its MFMA; the asm
  // statements order every accumulator read after the s_nop block.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i) asm volatile("" : "+a"(acc[j][i]));
  __syncthreads();  // every wave is done with the rings

  // Partial tile (token block i, channel block j) of wave v goes to slot q =
  // i' TN + j of wave v's part of the rings (i' = the rank of i among the
  // token blocks other than v), 1 KiB per slot, kPerArr slots per stage
  // object.
  auto slot_ptr = [&](int v, int q) -> uint8_t* {
    const int arr = q / C::kPerArr;
    uint8_t* base = arr == 0 ? ks0 : (arr == 1 ? ks1 : ks2);
    return base + v * C::kStage + (q % C::kPerArr) * 1024 + lane * 16;
  };
  auto hand_over = [&](auto vc) {
    constexpr int V = decltype(vc)::value;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i == V) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j)
        *reinterpret_cast<f32x4_t*>(slot_ptr(V, (i - (i > V ? 1 : 0)) * TN + j)) = acc[j][i];
    }
  };
  switch (wave) {
    case 0: hand_over(std::integral_constant<int, 0>{}); break;
    case 1: hand_over(std::integral_constant<int, 1>{}); break;
    case 2: hand_over(std::integral_constant<int, 2>{}); break;
    default: hand_over(std::integral_constant<int, 3>{}); break;
  }
  __syncthreads();

  // Wave w: token block w.  Lane (g, l16) of MFMA tile j holds channels
  // n0 + 16 j + 4 g + e (e = 0..3) of token m0 + 16 w + l16.  The decode
  // produced 2 T, so y = bf16(f(acc * (s / 2) + b)); (acc * (s / 2)) rounds
  // like (acc * s) / 2 except where a result is subnormal.
  auto finish = [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    const int row = m0 + 16 * W + l16;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      f32x4_t v = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int src = 0; src < 4; ++src) {
        if (src == W)
          v += acc[j][W];
        else
          v += *reinterpret_cast<const f32x4_t*>(slot_ptr(src, (W - (W > src ? 1 : 0)) * TN + j));
      }
      const int nb = n0 + 16 * j + 4 * g;
      const bool whole = nb + 3 < n;
      v *= unit ? f32x4_t{0.5f, 0.5f, 0.5f, 0.5f} : sc[j] * 0.5f;
      if constexpr (EPI) {
        v += bv[j];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (nb + e >= act_from) v[e] = gelu_tanh_f32(v[e]);
      }
      if (row < m) {
        uint16_t* yr = y + static_cast<int64_t>(row) * ldy + nb;
        if (whole && (y_flags & 1)) {
          u32x2_t o;
          o[0] = ks_pack_bf16x2(v[0], v[1]);
          o[1] = ks_pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<u32x2_t*>(yr) = o;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (nb + e < n) yr[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[e]));
        }
      }
    }
  };
  switch (wave) {
    case 0: finish(std::integral_constant<int, 0>{}); break;
    case 1: finish(std::integral_constant<int, 1>{}); break;
    case 2: finish(std::integral_constant<int, 2>{}); break;
    default: finish(std::integral_constant<int, 3>{}); break;
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// Bytes that the 8 XCDs fetch when the logical tiles are dealt to them in
// contiguous ranges (ks_logical_tile), in token-major or channel-major
// (col) order, each XCD reading the X rows of every token block and the
// weight rows of every channel tile in its range once into its own L2.
int64_t ks_fetch_estimate(int tiles_m, int tiles_n, int64_t x_block, int64_t w_block, bool col) {
  const int grid = tiles_m * tiles_n;
  const int minor = col ? tiles_m : tiles_n;
  int64_t total = 0;
  for (int xcd = 0; xcd < 8; ++xcd) {
    const int lo = xcd * (grid / 8) + (xcd < grid % 8 ? xcd : grid % 8);
    const int hi = lo + grid / 8 + (xcd < grid % 8 ? 1 : 0);
    if (hi <= lo) continue;
    const int majors = (hi - 1) / minor - lo / minor + 1;
    int minors = minor;
    if (majors == 1) {
      minors = hi - lo;
    } else if (majors == 2) {
      const int span = (minor - lo % minor) + ((hi - 1) % minor + 1);
      minors = span < minor ? span : minor;
    }
    total += (col ? minors : majors) * x_block + (col ? majors : minors) * w_block;
  }
  return total;
}

template <int TN, bool EPI>
hipError_t launch_ks(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const uint8_t* p,
                     int64_t n, int64_t ldp, const float* s, const float* bias, int act_from,
                     uint16_t* y, int64_t ldy, hipStream_t stream) {
  using C = KsCfg<TN>;
  const int tiles_m = static_cast<int>((m + C::kBM - 1) / C::kBM);
  const int tiles_n = static_cast<int>((n + C::kBN - 1) / C::kBN);
  // Channel-major order where it fetches fewer bytes: layers whose weights
  // outweigh their X (a few token blocks on a wide weight), so that the token
  // blocks of a channel tile share its weight rows in one L2.
  const int64_t x_block = int64_t{C::kBM} * k * 2;
  const int64_t w_block = int64_t{C::kBN} * k / 4;
  const bool col = ks_fetch_estimate(tiles_m, tiles_n, x_block, w_block, true) <
                   ks_fetch_estimate(tiles_m, tiles_n, x_block, w_block, false);
  const int y_flags = (((reinterpret_cast<uintptr_t>(y) & 7) == 0 && ldy % 4 == 0) ? 1 : 0) |
                      (col ? 2 : 0);
  hipLaunchKernelGGL((gemm_ternary_ksplit<TN, EPI>), dim3(static_cast<unsigned>(tiles_m) * tiles_n),
                     dim3(kKsThreads), 0, stream, reinterpret_cast<const uint8_t*>(x),
                     static_cast<int>(m), static_cast<int>(k), static_cast<int>(ldx), p,
                     static_cast<int>(n), static_cast<int>(ldp), s, bias, act_from, y,
                     static_cast<int>(ldy), tiles_n, y_flags);
  return hipGetLastError();
}

// Channels per tile (16 TN) for a layer, or 0 when the K-split kernel does
// not take it: the narrowest of 96, 144 and 192 channels whose 64-token tiles
// fill the chip at most once (a workgroup holds 120-144 KiB of LDS, so one
// runs per CU and a 257th tile would start a second round; a CU's work grows
// with the tile width), for K of at least 32 steps (with 4 steps a wave the
// three-stage prologue and the hand-over outweigh the split: 14.4 against
// 12.3 us with 64 x 128 tiles at M = 1024, K = 1024, N = 3072).  These are
// the layers whose larger tiles would leave CUs idle or whose 64 x 128
// tiles, K in sequence, leave each CU a long dependent stream.
int ksplit_channels_per_tile(int64_t m, int64_t k, int64_t n) {
  if (k < 2048) return 0;
  const int64_t tiles_m = (m + 63) / 64;
  for (const int tn : {6, 9, 12})
    if (tiles_m * ((n + 16 * tn - 1) / (16 * tn)) <= 256) return 16 * tn;
  return 0;
}

}  // namespace

bool gemm_ksplit_fits(int64_t m, int64_t k, int64_t n) {
  return ksplit_channels_per_tile(m, k, n) != 0;
}

hipError_t launch_gemm_ksplit(const uint16_t* x, int64_t m, int64_t k, int64_t ldx,
                              const uint8_t* p, int64_t n, int64_t ldp, const float* s,
                              const float* bias, int64_t act_from, uint16_t* y, int64_t ldy,
                              hipStream_t stream) {
  const int af = static_cast<int>(act_from);
  const bool epi = bias != nullptr || act_from < n;
  switch (ksplit_channels_per_tile(m, k, n)) {
    case 96:
      if (epi) return launch_ks<6, true>(x, m, k, ldx, p, n, ldp, s, bias, af, y, ldy, stream);
      return launch_ks<6, false>(x, m, k, ldx, p, n, ldp, s, nullptr, af, y, ldy, stream);
    case 144:
      if (epi) return launch_ks<9, true>(x, m, k, ldx, p, n, ldp, s, bias, af, y, ldy, stream);
      return launch_ks<9, false>(x, m, k, ldx, p, n, ldp, s, nullptr, af, y, ldy, stream);
    case 192:
      if (epi) return launch_ks<12, true>(x, m, k, ldx, p, n, ldp, s, bias, af, y, ldy, stream);
      return launch_ks<12, false>(x, m, k, ldx, p, n, ldp, s, nullptr, af, y, ldy, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace tern
