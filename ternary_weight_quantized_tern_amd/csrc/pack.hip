// 2-bit storage of ternary weights and its inverse.
//
// "1.58-bit FLUX" (arXiv 2412.18653), section 1: the 1.58-bit weights are
// stored as 2-bit signed integers, compressing them from 16 bits.  Layout
// (the reading used; the pages do not fix it): weight k of a row is the low
// two bits of its two's-complement value, in bits 2*(k%4) .. 2*(k%4)+1 of byte
// k/4 of the row.
//
// Both kernels are HBM-bound streams.  One thread handles one 16-weight group
// (16 int8 <-> one 32-bit word of codes) with 16-byte int8 accesses when the
// row pointer allows it; a grid-stride loop covers any n x k.  The flat group
// index is split into (row, group) with 32-bit arithmetic whenever every index
// the loop forms fits in 32 bits (all practical layer shapes), else 64-bit.
#include "internal.h"

namespace tern {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kMaxBlocks = 256 * 64;  // fills 256 CUs many times over

__device__ inline bool aligned_dev(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Four int8 values (one per byte of v) -> one byte of 2-bit codes.
__device__ inline uint32_t pack4(uint32_t v) {
  const uint32_t x = v & 0x03030303u;
  return (x | (x >> 6) | (x >> 12) | (x >> 18)) & 0xFFu;
}

// One byte of 2-bit codes -> four sign-extended int8 values (one per byte).
// The 2-bit fields are spread to the low bits of each byte, then a byte
// permute looks each one up in {00 -> 0, 01 -> 1, 10 -> -2, 11 -> -1}.
__device__ inline uint32_t unpack4(uint32_t b) {
  const uint32_t sel = (b | (b << 6) | (b << 12) | (b << 18)) & 0x03030303u;
  return __builtin_amdgcn_perm(0u, 0xFFFE0100u, sel);
}

template <typename IDX>
__global__ __launch_bounds__(kThreads) void pack_kernel(const int8_t* __restrict__ t, int64_t n,
                                                        int64_t k, int64_t ldt,
                                                        uint8_t* __restrict__ p, int64_t ldp) {
  const int64_t nbytes = (k + 3) / 4;
  const int64_t groups = (nbytes + 3) / 4;  // 16 weights per group
  const int64_t total = n * groups;
  const IDX groups_i = static_cast<IDX>(groups);
  for (IDX idx = static_cast<IDX>(blockIdx.x) * kThreads + threadIdx.x; idx < static_cast<IDX>(total);
       idx += static_cast<IDX>(gridDim.x) * kThreads) {
    const int64_t row = static_cast<int64_t>(idx / groups_i);
    const int64_t g = static_cast<int64_t>(idx - static_cast<IDX>(row) * groups_i);
    const int64_t k0 = g * 16;
    const int8_t* src = t + row * ldt + k0;
    uint32_t d[4];
    if (k0 + 16 <= k && aligned_dev(src, 16)) {
      const uint4 v = *reinterpret_cast<const uint4*>(src);
      d[0] = v.x;
      d[1] = v.y;
      d[2] = v.z;
      d[3] = v.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t kk = k0 + 4 * j + i;
          if (kk < k) w |= static_cast<uint32_t>(static_cast<uint8_t>(src[4 * j + i])) << (8 * i);
        }
        d[j] = w;
      }
    }
    const uint32_t word = pack4(d[0]) | (pack4(d[1]) << 8) | (pack4(d[2]) << 16) | (pack4(d[3]) << 24);
    uint8_t* dst = p + row * ldp + 4 * g;
    if (4 * g + 4 <= nbytes && aligned_dev(dst, 4)) {
      *reinterpret_cast<uint32_t*>(dst) = word;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * g + j < nbytes) dst[j] = static_cast<uint8_t>(word >> (8 * j));
    }
  }
}

template <typename IDX>
__global__ __launch_bounds__(kThreads) void unpack_kernel(const uint8_t* __restrict__ p, int64_t n,
                                                          int64_t k, int64_t ldp,
                                                          int8_t* __restrict__ t, int64_t ldt) {
  const int64_t nbytes = (k + 3) / 4;
  const int64_t groups = (nbytes + 3) / 4;
  const int64_t total = n * groups;
  const IDX groups_i = static_cast<IDX>(groups);
  for (IDX idx = static_cast<IDX>(blockIdx.x) * kThreads + threadIdx.x; idx < static_cast<IDX>(total);
       idx += static_cast<IDX>(gridDim.x) * kThreads) {
    const int64_t row = static_cast<int64_t>(idx / groups_i);
    const int64_t g = static_cast<int64_t>(idx - static_cast<IDX>(row) * groups_i);
    const uint8_t* src = p + row * ldp + 4 * g;
    uint32_t word = 0;
    if (4 * g + 4 <= nbytes && aligned_dev(src, 4)) {
      word = *reinterpret_cast<const uint32_t*>(src);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * g + j < nbytes) word |= static_cast<uint32_t>(src[j]) << (8 * j);
    }
    uint32_t d[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = unpack4((word >> (8 * j)) & 0xFFu);
    const int64_t k0 = g * 16;
    int8_t* dst = t + row * ldt + k0;
    if (k0 + 16 <= k && aligned_dev(dst, 16)) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(d[0], d[1], d[2], d[3]);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (k0 + j < k) dst[j] = static_cast<int8_t>(d[j / 4] >> (8 * (j % 4)));
    }
  }
}

// Transposed packing: the codes of p (row n, packed along k) packed along n
// into pt (row k holds T[0..n-1][k]).  A workgroup moves a tile of 128 rows
// of p by 128 bytes (512 codes), so that it reads whole 128-byte lines (a
// narrower tile leaves each line to several workgroups, which the round-robin
// placement puts on different XCDs, each fetching the line into its own L2).
// Load: 16-byte pieces of the tile rows into LDS (eight threads per row).
// Transpose: work item (c, q) takes byte column c (codes k = 4c .. 4c+3) of
// tile rows 16q .. 16q+15, splits the 16 bytes by field with shifts and
// masks, gathers the four 2-bit fields of each 4-byte group into one byte
// with a byte dot product against (1, 4, 16, 64), and writes 4 bytes (16 codes
// along n) into each of the rows 4c .. 4c+3 of pt.  Rows of the tile past n
// read as zero, so the fields past n in the last byte of a pt row are zero.
constexpr int kTRows = 128;            // rows of p (codes along n) per tile
constexpr int kTBytes = 128;           // bytes of p per tile row (512 codes along k)
constexpr int kTPitch = kTBytes + 4;   // LDS row pitch (bytes)
constexpr int kTLoads = kTRows * kTBytes / 16 / kThreads;       // 16-byte loads per thread
constexpr int kTGroups = kTRows / 16;                            // 16-row groups per tile
constexpr int kTItems = (kTBytes * kTGroups) / kThreads;        // (c, q) items per thread
static_assert(kTLoads * kThreads * 16 == kTRows * kTBytes && kTItems * kThreads == kTBytes * kTGroups,
              "whole loads and items per thread");

__global__ __launch_bounds__(kThreads) void pack_transposed_kernel(
    const uint8_t* __restrict__ p, int64_t n, int64_t k, int64_t ldp, uint8_t* __restrict__ pt,
    int64_t ldpt, int64_t tiles_k, bool p_vec, bool pt_vec) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTRows * kTPitch];
  const int64_t in_bytes = (k + 3) / 4;   // bytes of a p row
  const int64_t out_bytes = (n + 3) / 4;  // bytes of a pt row
  const int64_t tiles = ((n + kTRows - 1) / kTRows) * tiles_k;
  const int t = threadIdx.x;
  for (int64_t b = blockIdx.x; b < tiles; b += gridDim.x) {
    const int64_t tn = b / tiles_k;
    const int64_t n0 = tn * kTRows;
    const int64_t kb0 = (b - tn * tiles_k) * kTBytes;  // first byte column of p
    uint32_t w[kTLoads][4];
#pragma unroll
    for (int i = 0; i < kTLoads; ++i) {
      const int id = i * kThreads + t;
      const int r = id / (kTBytes / 16);
      const int64_t col = kb0 + 16 * (id % (kTBytes / 16));
#pragma unroll
      for (int e = 0; e < 4; ++e) w[i][e] = 0u;
      if (n0 + r < n) {
        const uint8_t* src = p + (n0 + r) * ldp + col;
        if (p_vec && col + 16 <= in_bytes) {
          const uint4 v = *reinterpret_cast<const uint4*>(src);
          w[i][0] = v.x;
          w[i][1] = v.y;
          w[i][2] = v.z;
          w[i][3] = v.w;
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (col + e < in_bytes) w[i][e / 4] |= static_cast<uint32_t>(src[e]) << (8 * (e % 4));
        }
      }
    }
    __syncthreads();  // the previous tile's reads are done
#pragma unroll
    for (int i = 0; i < kTLoads; ++i) {
      const int id = i * kThreads + t;
      const int r = id / (kTBytes / 16);
      const int c0 = 16 * (id % (kTBytes / 16));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<uint32_t*>(&tile[r * kTPitch + c0 + 4 * e]) = w[i][e];
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kTItems; ++it) {
      const int id = it * kThreads + t;
      const int c = id / kTGroups;  // byte column of the tile
      const int q = id % kTGroups;  // 16-row group
      uint32_t d[4];  // byte i of d[j]: tile row 16 q + 4 j + i, byte column c
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t v = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v |= static_cast<uint32_t>(tile[(16 * q + 4 * j + i) * kTPitch + c]) << (8 * i);
        d[j] = v;
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int64_t row = 4 * (kb0 + c) + f;  // row of pt (code column k of p)
        if (row >= k) break;
        uint32_t o = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t fields = (d[j] >> (2 * f)) & 0x03030303u;
          o |= __builtin_amdgcn_udot4(fields, 0x40100401u, 0u, false) << (8 * j);
        }
        const int64_t byte0 = n0 / 4 + 4 * q;
        uint8_t* dst = pt + row * ldpt + byte0;
        if (pt_vec && byte0 + 4 <= out_bytes) {
          *reinterpret_cast<uint32_t*>(dst) = o;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (byte0 + j < out_bytes) dst[j] = static_cast<uint8_t>(o >> (8 * j));
        }
      }
    }
  }
}

inline unsigned grid_for(int64_t work_items) {
  int64_t blocks = (work_items + kThreads - 1) / kThreads;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  if (blocks < 1) blocks = 1;
  return static_cast<unsigned>(blocks);
}

// The loop's indices stay below total + (grid size) * kThreads, the grid
// being at most kMaxBlocks workgroups.
inline bool fits_u32(int64_t total) {
  return total + kMaxBlocks * kThreads < (int64_t(1) << 32);
}

}  // namespace

hipError_t launch_pack(const int8_t* t, int64_t n, int64_t k, int64_t ldt, uint8_t* p,
                       int64_t ldp, hipStream_t stream) {
  const int64_t groups = ((k + 3) / 4 + 3) / 4;
  const dim3 grid(grid_for(n * groups));
  if (fits_u32(n * groups))
    hipLaunchKernelGGL(pack_kernel<uint32_t>, grid, dim3(kThreads), 0, stream, t, n, k, ldt, p, ldp);
  else
    hipLaunchKernelGGL(pack_kernel<uint64_t>, grid, dim3(kThreads), 0, stream, t, n, k, ldt, p, ldp);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* p, int64_t n, int64_t k, int64_t ldp, int8_t* t,
                         int64_t ldt, hipStream_t stream) {
  const int64_t groups = ((k + 3) / 4 + 3) / 4;
  const dim3 grid(grid_for(n * groups));
  if (fits_u32(n * groups))
    hipLaunchKernelGGL(unpack_kernel<uint32_t>, grid, dim3(kThreads), 0, stream, p, n, k, ldp, t, ldt);
  else
    hipLaunchKernelGGL(unpack_kernel<uint64_t>, grid, dim3(kThreads), 0, stream, p, n, k, ldp, t, ldt);
  return hipGetLastError();
}

hipError_t launch_pack_transposed(const uint8_t* p, int64_t n, int64_t k, int64_t ldp,
                                  uint8_t* pt, int64_t ldpt, hipStream_t stream) {
  const int64_t tiles_k = ((k + 3) / 4 + kTBytes - 1) / kTBytes;
  int64_t tiles = ((n + kTRows - 1) / kTRows) * tiles_k;
  if (tiles > kMaxBlocks) tiles = kMaxBlocks;
  const bool p_vec = reinterpret_cast<uintptr_t>(p) % 16 == 0 && ldp % 16 == 0;
  const bool pt_vec = reinterpret_cast<uintptr_t>(pt) % 4 == 0 && ldpt % 4 == 0;
  hipLaunchKernelGGL(pack_transposed_kernel, dim3(static_cast<unsigned>(tiles)), dim3(kThreads),
                     0, stream, p, n, k, ldp, pt, ldpt, tiles_k, p_vec, pt_vec);
  return hipGetLastError();
}

}  // namespace tern
