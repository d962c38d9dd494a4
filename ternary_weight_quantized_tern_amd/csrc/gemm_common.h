// Device helpers shared by the ternary GEMM kernels (gemm.hip, gemm_small.hip):
// vector types, raw buffer resources, the 2-bit code -> bf16 decode and the
// tied-accumulator bf16 and int8 MFMAs.  Internal to libternary.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tern {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((address_space(3))) void lds_void_t;

inline constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), static_cast<int>(kRsrcWord3));
}

// Sixteen 2-bit codes (code c in bits 2c..2c+1 of w) -> two MFMA operands
// of eight bf16 values 0 / +2 / -2 in ascending k: `lo` gets codes 0..7, `hi`
// codes 8..15.  t[r] = (w << (6 - 2r)) & 0xC0C0C0C0 holds code 4b + r in bits
// 6..7 of byte b with zeros below: the high byte of that code's bf16 value
// (00 -> 0x00, 01 -> 0x40 = +2, 11 -> 0xC0 = -2).  A byte permute puts two
// such bytes over zero low bytes: operand register q of block h holds codes
// 8h + 2q and 8h + 2q + 1.  15 VALU instructions for 16 codes.
__device__ inline void decode16(uint32_t w, bf16x8_t& lo, bf16x8_t& hi) {
  uint32_t t[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) t[r] = (w << (6 - 2 * r)) & 0xC0C0C0C0u;
  u32x4_t a, b;
  a[0] = __builtin_amdgcn_perm(t[1], t[0], 0x040C000Cu);
  a[1] = __builtin_amdgcn_perm(t[3], t[2], 0x040C000Cu);
  a[2] = __builtin_amdgcn_perm(t[1], t[0], 0x050C010Cu);
  a[3] = __builtin_amdgcn_perm(t[3], t[2], 0x050C010Cu);
  b[0] = __builtin_amdgcn_perm(t[1], t[0], 0x060C020Cu);
  b[1] = __builtin_amdgcn_perm(t[3], t[2], 0x060C020Cu);
  b[2] = __builtin_amdgcn_perm(t[1], t[0], 0x070C030Cu);
  b[3] = __builtin_amdgcn_perm(t[3], t[2], 0x070C030Cu);
  lo = __builtin_bit_cast(bf16x8_t, a);
  hi = __builtin_bit_cast(bf16x8_t, b);
}

// One v_mfma_f32_16x16x32_bf16 with the accumulator tied to the same
// AGPRs on input and output (ZERO: C is the constant 0).  Written as inline
// asm because the compiler's own form of this loop copies accumulators
// between AGPRs with v_accvgpr_mov, which costs about a quarter of the
// matrix-core throughput.  The compiler does not see the MFMA inside, so the
// caller keeps its hazards: an MFMA may read a VGPR only two wait states
// after a VALU instruction wrote it.  PAD puts an s_nop 1 in front of the
// MFMA for that; a caller whose schedule keeps every VALU-written operand
// further away passes PAD = false (each s_nop 1 costs issue cycles that the
// MFMA stream does not hide).
template <bool ZERO, bool PAD = true>
__device__ inline void mfma16(f32x4_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  if constexpr (ZERO && PAD) {
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
  } else if constexpr (ZERO) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
  } else if constexpr (PAD) {
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  } else {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  }
}

// One v_mfma_i32_16x16x64_i8 (16 int8 values per lane and operand, exact
// int32 sums), tied like mfma16.  The accumulator registers are declared
// fp32 and hold the int32 sums as bit patterns; the same hazard rule holds.
template <bool ZERO, bool PAD = true>
__device__ inline void mfma_i8(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b) {
  if constexpr (ZERO && PAD) {
    asm volatile("s_nop 1\n\tv_mfma_i32_16x16x64_i8 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
  } else if constexpr (ZERO) {
    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
  } else if constexpr (PAD) {
    asm volatile("s_nop 1\n\tv_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  } else {
    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  }
}

// The MFMA of an operand kind: int8 (A8) or bf16, operands as raw registers.
template <bool A8, bool ZERO, bool PAD>
__device__ inline void mfma_op(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b) {
  if constexpr (A8)
    mfma_i8<ZERO, PAD>(acc, a, b);
  else
    mfma16<ZERO, PAD>(acc, __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b));
}

// The tanh form of GELU (Hendrycks and Gimpel) in fp32:
//   gelu(z) = z/2 (1 + tanh u),  u = sqrt(2/pi) (z + 0.044715 z^3).
// Since (1 + tanh u)/2 = 1/(1 + e^(-2u)), gelu(z) = z / (1 + e^(-2u)): the
// denominator is at least 1 (no cancellation for negative z), e^(-2u) = 2^a
// with a = z (A + B z^2), A = -2 sqrt(2/pi) log2 e, B = 0.044715 A, and an
// overflow to +inf gives the limit 0.  Five VALU instructions, the hardware
// exp2 and one hardware reciprocal.
__device__ inline float gelu_tanh_f32(float z) {
  constexpr float kA = -2.302208198144325f;    // -2 sqrt(2/pi) log2(e)
  constexpr float kB = -0.1029432395800235f;   // 0.044715 kA
  const float a = z * __builtin_fmaf(kB, z * z, kA);
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a));
}

}  // namespace tern
