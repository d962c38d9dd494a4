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
// s_waitcnt immediate that waits until at most n vector memory operations
// are outstanding (expcnt and lgkmcnt not waited for).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) & 3) << 14; }

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

// bf16 activations, a handful of tokens: the weight stream with every load of
// a wave in flight at once.  A workgroup owns RB blocks of 16 output channels
// and all of K; its W waves (W = blockDim.x / 64, at most 16) split K in
// 256-wide chunks, wave w taking chunks w, w + W, w + 2 W, ...  In each round
// a wave issues the loads of its next CPW chunks together (the chunk loop is
// unrolled): first the X copies of every chunk, then the weight words chunk
// by chunk, so that it can decode each chunk's codes as soon as that chunk's
// words have landed (the loads complete in issue order) while the later
// ones are still in flight, accumulating R blocks of 16 tokens.  Without
// LOOP one round covers all of K.  MAXW bounds the waves
// per workgroup (and so sets the register budget: 128 per lane at 16 waves,
// 256 at 8).
//
// Lane (r, g) fetches 16 bytes of weight row r of every channel block per
// chunk (codes 64 g .. 64 g + 63 of the chunk); MFMA (d, h) of a chunk uses
// codes 16 d + 8 h .. 16 d + 8 h + 7 of those 64, i.e. the 16-byte piece
// 8 g + 2 d + h of the chunk's 256 X values of token r (the same permutation
// of k on both operands).  Loaded straight into registers, those X pieces
// would be 64 lanes touching 64 different cache lines per load instruction,
// which keeps the texture addresser busy for most of the kernel; instead each
// wave copies the X rows of its chunk (only the real tokens, rounded up to
// two) into its own LDS region with buffer loads in the LDS-DMA form, 512
// contiguous bytes per row, and reads the MFMA operands from there.  The
// 16-byte pieces of LDS row r are XOR-swizzled by r % 16 (applied on the
// global side of the copy), so that an operand read of 16 token rows hits 16
// distinct bank groups; operand lanes of tokens past the copied rows read
// row 0 (their outputs are not stored).
//
// Chunk slots past the last chunk copy no X and skip their decode (a
// wave-uniform branch) but still load their weight words, which lie past k
// and read as zero, so that exactly CPW * RB weight loads follow the copies;
// the 64-code pieces past k, weight rows past n and tokens past m read as
// zero through the buffer range check.  The partial sums of the W waves meet in
// LDS (in the X regions, after a barrier); channel block bl is finished by
// wave bl % W, which adds the partials in wave order, applies the fp32
// channel scale (and the optional bias and tanh-form GELU) and rounds once to
// bf16, so the blocks' epilogues run in parallel.
// The MFMAs are the compiler's builtin, so that the compiler sees their
// latencies (with a chunk slot that may be skipped, it moves accumulators
// between registers at the join, and only a visible MFMA makes it wait for
// the result before such a move).  p is not declared __restrict__: with it
// the compiler takes the weight loads for invariant and may move them past
// the wait for the X copies (or into the conditional decode), where that
// wait would no longer cover the copies.
template <int RB, int R, int CPW, int MAXW, bool EPI, bool LOOP>
__global__ __launch_bounds__(64 * MAXW) void gemm_ternary_few(
    const uint8_t* __restrict__ x, int m, int k, int ldx, const uint8_t* p, int n,
    int ldp, const float* __restrict__ s, const float* __restrict__ bias, int act_from,
    uint16_t* __restrict__ y, int ldy, int y_vec_ok) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(CPW * RB < 64, "the wait for the X copies counts CPW * RB loads");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem_few[];

  const int waves = blockDim.x >> 6;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int n0 = blockIdx.x * (16 * RB);
  const int rows = (n - n0) < 16 * RB ? (n - n0) : 16 * RB;
  // X rows copied per chunk (the real tokens, rounded up to two) and their
  // LDS bytes; the LDS region of slot i of this wave.
  const int mrows = (m < 16 * R ? m : 16 * R) + 1 & ~1;
  const uint32_t region = static_cast<uint32_t>(mrows) * 512u;

  const __amdgpu_buffer_rsrc_t prs = make_rsrc(
      p + static_cast<int64_t>(n0) * ldp, static_cast<uint32_t>((rows - 1) * ldp + k / 4));
  const __amdgpu_buffer_rsrc_t xrs =
      make_rsrc(x, static_cast<uint32_t>((static_cast<int64_t>(m) - 1) * ldx * 2 + k * 2));
  const int chunks = (k + kChunk - 1) / kChunk;

  const uint32_t p_off = static_cast<uint32_t>(r16 * ldp + 16 * g);
  // Copy plan: copy d of a chunk moves rows 2 d and 2 d + 1; lane l fills the
  // 16-byte slot l % 32 of row 2 d + l / 32, which holds piece slot ^ (row %
  // 16) of the row's chunk.
  const uint32_t crow = static_cast<uint32_t>(lane >> 5);
  const uint32_t cslot = static_cast<uint32_t>(lane & 31);
  // Operand reads: token row r (tokens past the copied rows read row 0),
  // piece (8 g + j) ^ (r % 16) for j = 2 d + h.
  uint32_t rd_row[R], rd_x[R];
#pragma unroll
  for (int b = 0; b < R; ++b) {
    const int r = 16 * b + r16;
    const int rc = r < mrows ? r : 0;
    rd_row[b] = static_cast<uint32_t>(rc) * 512u;
    rd_x[b] = static_cast<uint32_t>(8 * g) ^ static_cast<uint32_t>(rc & 15);
  }

  // Channel block bl of the output is finished by wave bl % waves.  That wave
  // requests the block's channel scales (and biases) before the weight
  // stream, so that they have arrived by the epilogue: one 16-byte buffer load
  // per block and lane (four consecutive channels), without a per-lane branch
  // (the range check is per 4-byte word: channels past n, and a null vector,
  // read as zero).  A null scale vector means unit scales (the input-gradient
  // product).
  const bool unit = s == nullptr;
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(unit ? p : reinterpret_cast<const uint8_t*>(s + n0),
                unit ? 0u : static_cast<uint32_t>(rows * 4));
  const __amdgpu_buffer_rsrc_t brs =
      make_rsrc(bias == nullptr ? p : reinterpret_cast<const uint8_t*>(bias + n0),
                (!EPI || bias == nullptr) ? 0u : static_cast<uint32_t>(rows * 4));
  f32x4_t sraw[RB];
  f32x4_t braw[EPI ? RB : 1];
#pragma unroll
  for (int bl = 0; bl < RB; ++bl) {
    sraw[bl] = f32x4_t{};
    if constexpr (EPI) braw[bl] = f32x4_t{};
    if (bl % waves == wave) {
      const uint32_t off = static_cast<uint32_t>((16 * bl + 4 * g) * 4);
      sraw[bl] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(srs, off, 0, 0));
      if constexpr (EPI)
        braw[bl] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(brs, off, 0, 0));
    }
  }

  f32x4_t acc[RB][R];
#pragma unroll
  for (int bl = 0; bl < RB; ++bl)
#pragma unroll
    for (int b = 0; b < R; ++b) acc[bl][b] = f32x4_t{};

  for (int base = 0; base < chunks; base += waves * CPW) {
    // The X rows of every live slot first ...
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = base + wave + waves * i;
      if (c < chunks) {
        const uint32_t dst = static_cast<uint32_t>((wave * CPW + i)) * region;
#pragma unroll
        for (int d = 0; d < 8 * R; ++d) {
          if (2 * d >= mrows) break;
          const uint32_t row = 2u * d + crow;
          const uint32_t piece = cslot ^ (row & 15u);
          const uint32_t kp = static_cast<uint32_t>(c * kChunk) + 8u * piece;
          const uint32_t poob = (static_cast<uint32_t>(k - 1) - kp) & kOutOfRange;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              xrs, (lds_void_t*)(smem_few + dst + 1024u * d), 16,
              (row * static_cast<uint32_t>(ldx) * 2u + 2u * kp) | poob, 0, 0, 0);
        }
      }
    }
    asm volatile("" ::: "memory");
    // ... then the weight words of every slot in slot order (a slot past the
    // last chunk reads zeros: its codes lie past k), so that CPW * RB loads
    // always follow the copies.
    u32x4_t wq[CPW][RB];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = base + wave + waves * i;
      const int kc = c * kChunk + 64 * g;
      const uint32_t oob = static_cast<uint32_t>(k - 1 - kc) & kOutOfRange;
#pragma unroll
      for (int bl = 0; bl < RB; ++bl)
        wq[i][bl] = __builtin_bit_cast(
            u32x4_t,
            __builtin_amdgcn_raw_buffer_load_b128(
                prs, (p_off + static_cast<uint32_t>(bl * 16 * ldp + c * (kChunk / 4))) | oob, 0,
                0));
    }
    // The copies have landed once at most CPW * RB loads are outstanding; the
    // weight words are waited for one by one where they are decoded.  (The
    // empty asm statements keep the loads before the wait and the LDS reads
    // after it.)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPW * RB));
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      if (base + wave + waves * i < chunks) {
        const uint8_t* xl = smem_few + static_cast<uint32_t>((wave * CPW + i)) * region;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          // The two X operands of code word d (pieces 2 d and 2 d + 1), each
          // feeding RB blocks of MFMAs.
          bf16x8_t xo[2][R];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b = 0; b < R; ++b)
              xo[h][b] = *reinterpret_cast<const bf16x8_t*>(
                  xl + rd_row[b] + 16u * (rd_x[b] ^ static_cast<uint32_t>(2 * d + h)));
#pragma unroll
          for (int bl = 0; bl < RB; ++bl) {
            bf16x8_t lo, hi;
            decode16(wq[i][bl][d], lo, hi);
#pragma unroll
            for (int b = 0; b < R; ++b) {
              acc[bl][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, xo[0][b], acc[bl][b], 0, 0, 0);
              acc[bl][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, xo[1][b], acc[bl][b], 0, 0, 0);
            }
          }
        }
      }
    }
    if constexpr (!LOOP) break;
    // Only the loads of slots past the last chunk (zeros) can still be in
    // flight; with none left, the next round's copies and loads need not
    // wait for them before reusing their registers.  The next round refills
    // the regions: every wave must be done reading.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
  }

  // The partial sums of the waves meet in LDS (in the X regions, free once
  // every wave is past its last read): [waves][RB][R][64] sums of 4 channels.
  // Wave bl % waves then adds, for channel block bl, the partials in wave
  // order 0, 1, 2, ... (a fixed order: repeated calls give identical bits),
  // applies the scale (and bias and GELU) and stores the block's outputs.
  f32x4_t* red = reinterpret_cast<f32x4_t*>(smem_few);
  if (waves > 1) {
    __syncthreads();
#pragma unroll
    for (int bl = 0; bl < RB; ++bl)
#pragma unroll
      for (int b = 0; b < R; ++b) red[((wave * RB + bl) * R + b) * 64 + lane] = acc[bl][b];
    __syncthreads();
  }

#pragma unroll
  for (int bl = 0; bl < RB; ++bl) {
    if (bl % waves != wave) continue;
    const int nb = n0 + 16 * bl + 4 * g;  // output channels nb .. nb + 3 of this lane
#pragma unroll
    for (int b = 0; b < R; ++b) {
      f32x4_t v = acc[bl][b];
      if (waves > 1) {
        // Partials read four at a time ahead of their (ordered) additions.
        v = red[(bl * R + b) * 64 + lane];
        for (int w0 = 1; w0 < waves; w0 += 4) {
          f32x4_t t[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int w = (w0 + i < waves) ? w0 + i : waves - 1;
            t[i] = red[((w * RB + bl) * R + b) * 64 + lane];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (w0 + i < waves) v += t[i];
        }
      }
      const int token = 16 * b + r16;
      if (token >= m) continue;
      __bf16 o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // The decode produced 2 T: y = bf16(acc * (s / 2)), which rounds like
        // bf16(fp32(acc / 2 * s)) (the halving is exact).
        float z = v[e] * ((unit ? 1.0f : sraw[bl][e]) * 0.5f);
        if constexpr (EPI) {
          z += braw[bl][e];
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
#endif  // __HIP_DEVICE_COMPILE__
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

// LDS of a few-token launch: the X regions (waves * CPW chunks of the copied
// token rows, 512 bytes each), reused for the partial sums of every wave.
constexpr int64_t kFewLdsMax = 96 * 1024;

template <int RB, int R, int CPW, int MAXW, bool EPI>
hipError_t launch_few(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const uint8_t* p,
                      int64_t n, int64_t ldp, const float* s, const float* bias, int act_from,
                      uint16_t* y, int64_t ldy, hipStream_t stream) {
  const int64_t blocks = (n + 16 * RB - 1) / (16 * RB);
  const int64_t chunks = (k + kChunk - 1) / kChunk;
  const int64_t mrows = ((m < 16 * R ? m : 16 * R) + 1) & ~int64_t{1};
  // Waves: enough for one round over K with CPW chunks each, at most MAXW
  // and at most what the LDS budget holds.
  int64_t waves = (chunks + CPW - 1) / CPW;
  if (waves > MAXW) waves = MAXW;
  const int64_t by_lds = kFewLdsMax / (CPW * mrows * 512);
  if (waves > by_lds) waves = by_lds;
  if (waves < 1) waves = 1;
  const int64_t x_lds = waves * CPW * mrows * 512;
  const int64_t red_lds = waves * RB * R * 64 * static_cast<int64_t>(sizeof(f32x4_t));
  const size_t lds = static_cast<size_t>(x_lds > red_lds ? x_lds : red_lds);
  const int y_vec_ok = ((reinterpret_cast<uintptr_t>(y) & 7) == 0) && (ldy % 4 == 0);
  const dim3 grid(static_cast<unsigned>(blocks)), block(static_cast<unsigned>(64 * waves));
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
  if (chunks <= waves * CPW)
    hipLaunchKernelGGL((gemm_ternary_few<RB, R, CPW, MAXW, EPI, false>), grid, block, lds, stream, xb,
                       static_cast<int>(m), static_cast<int>(k), static_cast<int>(ldx), p,
                       static_cast<int>(n), static_cast<int>(ldp), s, bias, act_from, y,
                       static_cast<int>(ldy), y_vec_ok);
  else
    hipLaunchKernelGGL((gemm_ternary_few<RB, R, CPW, MAXW, EPI, true>), grid, block, lds, stream, xb,
                       static_cast<int>(m), static_cast<int>(k), static_cast<int>(ldx), p,
                       static_cast<int>(n), static_cast<int>(ldp), s, bias, act_from, y,
                       static_cast<int>(ldy), y_vec_ok);
  return hipGetLastError();
}

// Shape of the few-token launch, from a sweep of the FLUX and DiT layer
// shapes at 1 to 32 tokens (graph replays over a 1 GiB pool of distinct
// weights).  Each X operand read from LDS feeds RB channel blocks of MFMAs
// and every workgroup copies the X rows of all of K, so RB grows with the
// tokens as long as the layer still gives enough workgroups:
//  * at most 4 tokens (X is cheap): two blocks and three chunks per wave on
//    the largest layers (at least 1024 blocks), else one block and two
//    chunks per wave, up to 16 waves;
//  * 5 to 16 tokens: six blocks (one chunk per wave, up to 16 waves) with
//    more than 8 tokens where that still gives 224 workgroups; else three
//    blocks and three chunks per wave from 384 blocks (up to 8 waves); two
//    blocks from 256; one block (two chunks per wave past 16 chunks);
//  * 17 to 32 tokens (two MFMA row blocks, up to 8 waves for the
//    registers): six blocks from 1344, three from 384, two from 256, else
//    one, one chunk per wave (two past 16 chunks on one block).
template <bool EPI>
hipError_t launch_few_any(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const uint8_t* p,
                          int64_t n, int64_t ldp, const float* s, const float* bias, int act_from,
                          uint16_t* y, int64_t ldy, hipStream_t stream) {
  const int64_t nb = (n + 15) / 16;
  const int64_t chunks = (k + kChunk - 1) / kChunk;
#define TERN_FEW(RB, R, CPW, MAXW) \
  return launch_few<RB, R, CPW, MAXW, EPI>(x, m, k, ldx, p, n, ldp, s, bias, act_from, y, ldy, stream);
  if (m <= 4) {
    if (nb >= 1024) TERN_FEW(2, 1, 3, 8)
    TERN_FEW(1, 1, 2, 16)
  }
  if (m <= 16) {
    if (m > 8 && nb >= 6 * 224) TERN_FEW(6, 1, 1, 16)
    if (nb >= 384) TERN_FEW(3, 1, 3, 8)
    if (nb >= 256) TERN_FEW(2, 1, 1, 16)
    if (chunks > 16) TERN_FEW(1, 1, 2, 16)
    TERN_FEW(1, 1, 1, 16)
  }
  if (nb >= 6 * 224) TERN_FEW(6, 2, 1, 8)
  if (nb >= 384) TERN_FEW(3, 2, 1, 8)
  if (nb >= 256) TERN_FEW(2, 2, 1, 8)
  if (chunks > 16) TERN_FEW(1, 2, 2, 8)
  TERN_FEW(1, 2, 1, 8)
#undef TERN_FEW
}

}  // namespace

hipError_t launch_gemm_small(const uint16_t* x, int64_t m, int64_t k, int64_t ldx,
                             const uint8_t* p, int64_t n, int64_t ldp, const float* s,
                             const float* bias, int64_t act_from, uint16_t* y, int64_t ldy,
                             hipStream_t stream) {
  if (bias != nullptr || act_from < n)
    return launch_few_any<true>(x, m, k, ldx, p, n, ldp, s, bias, static_cast<int>(act_from), y,
                                ldy, stream);
  return launch_few_any<false>(x, m, k, ldx, p, n, ldp, s, nullptr, static_cast<int>(act_from), y,
                               ldy, stream);
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
