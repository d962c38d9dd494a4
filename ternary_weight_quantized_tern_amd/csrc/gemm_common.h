// Device helpers shared by the ternary GEMM kernels (gemm.hip, gemm_small.hip):
// vector types, raw buffer resources, the 2-bit code -> bf16 decode and the
// tied-accumulator bf16 MFMA.  Internal to libternary.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tern {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((address_space(3))) void lds_void_t;

inline constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), static_cast<int>(kRsrcWord3));
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

// One v_mfma_f32_16x16x32_bf16 with the accumulator tied to the same
// AGPRs on input and output (ZERO: C is the constant 0).  Written as inline
// asm because the compiler's own form of this loop copies accumulators
// between AGPRs with v_accvgpr_mov, which costs about a quarter of the
// matrix-core throughput.  The compiler does not see the MFMA inside, so the
// asm keeps its hazards itself: the leading s_nop 1 gives the two wait states
// that a VALU write of an A or B operand needs before an MFMA reads it (the
// decoded weights are VALU results).
template <bool ZERO>
__device__ inline void mfma16(f32x4_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  if constexpr (ZERO) {
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
  } else {
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  }
}

}  // namespace tern
