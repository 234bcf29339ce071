// Helpers of the bf16 prefill kernel (fwd_bf16.hip).
#pragma once

#include "attn_common.h"

namespace attn {
namespace prefill {

// xor swizzle of the 16-byte chunk index of V row r inside a row-major LDS tile: the
// transpose reads of a half wave (4 rows x 64 bytes) then touch 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  if constexpr (D == 128) return 4 * (r & 3);
  else return 4 * ((r >> 1) & 1);
}

// (c, s) <- (c, s) rotated by the angle whose cosine and sine are (sc, ss).
__device__ __forceinline__ void cmul(float& c, float& s, float sc, float ss) {
  const float nc = c * sc - s * ss;
  const float ns = c * ss + s * sc;
  c = nc;
  s = ns;
}

// Smallest value >= x (finite) whose significand has at most 16 bits: such a value is the
// exact sum of two bf16 numbers (its top 8 bits and the rest), so it can be subtracted
// inside a bf16 matrix product exactly.
__device__ __forceinline__ float ceil_sig16(float x) {
  uint32_t r = __builtin_bit_cast(uint32_t, x) & 0xffffff00u;
  if (__builtin_bit_cast(float, r) < x) r += 0x100u;  // only for x > 0 (truncation rounds down)
  return __builtin_bit_cast(float, r);
}

// The two bf16 pieces (hi in the low half, lo in the high half) of a value with a 16-bit
// significand, packed for one MFMA operand dword: hi + lo == v exactly.
__device__ __forceinline__ uint32_t split_bf16_pair(float v) {
  const uint32_t hb = __builtin_bit_cast(uint32_t, v) & 0xffff0000u;
  const float lo = v - __builtin_bit_cast(float, hb);  // exact: at most 8 significant bits
  return (hb >> 16) | (__builtin_bit_cast(uint32_t, lo) & 0xffff0000u);
}

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

}  // namespace prefill
}  // namespace attn
