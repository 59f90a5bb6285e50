// skv_mfma.h -- v_mfma_f32_16x16x32_bf16 operand helpers (gfx950).
//
// Lane layout of the 16x16x32 bf16 MFMA (64 lanes, q = lane / 16, i = lane % 16):
//   A (16 x 32): lane holds A[i][8q .. 8q+7]
//   B (32 x 16): lane holds B[8q .. 8q+7][i]
//   C (16 x 16): lane holds C[4q + r][i] for r = 0..3
// so an operand whose reduction index runs along memory (a K row, a Q row) is
// one 16-byte load per lane.
#pragma once
#include "skv_common.h"

namespace skv {

__device__ __forceinline__ floatx4_t mfma_bf16(const bf16x8_t& a, const bf16x8_t& b, const floatx4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace skv
