// The append into an 8-bit (OCP E4M3) cache with one fp32 scale per (block, KV head), shared by
// the append kernel and by the decode kernel that fuses the append into its launch, so that both
// produce the same codes and scales bit for bit.
//
// The pages say only that the KV cache may be kept in 8 bits ("serving-paged-attention", section
// "실무에서 만지는 지점"). The scale is kept an upper bound of the block's content over 448:
//   s_prev = scale[blk, h], or 0 when the token is the block's first (offset 0);
//   a = max |x| over the token's row; s = a / 448 if a > s_prev * 448 else s_prev; s = 1 if 0;
//   if s changed and earlier tokens exist, their codes c become enc((dec(c) * s_prev) / s);
//   the token is stored as enc(x / s); enc clamps to +-448 and rounds to nearest-even.
// All arithmetic is fp32 with IEEE division.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pa {

typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float e4m3_max() { return 448.f; }

// Clamp two floats to the E4M3 range and convert them, round-to-nearest-even, into bytes 0-1
// (HI = false) or 2-3 (HI = true) of `old`.
template <bool HI>
__device__ __forceinline__ uint32_t enc_pair(float a, float b, uint32_t old) {
  a = fminf(fmaxf(a, -e4m3_max()), e4m3_max());
  b = fminf(fmaxf(b, -e4m3_max()), e4m3_max());
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// The block's scale after appending a row whose largest magnitude is amax.
__device__ __forceinline__ float fp8_append_scale(float amax, float s_prev) {
  const float s = amax > s_prev * e4m3_max() ? amax / e4m3_max() : s_prev;
  return s == 0.f ? 1.f : s;
}

// An earlier token's decoded value expressed under the new scale (before encoding).
__device__ __forceinline__ float fp8_rescaled(float decoded, float s_prev, float s) {
  return (decoded * s_prev) / s;
}

// The four codes of a word re-encoded from scale s_prev to scale s.
__device__ __forceinline__ uint32_t fp8_reencode_word(uint32_t w, float s_prev, float s) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  const uint32_t o = enc_pair<false>(fp8_rescaled(lo.x, s_prev, s), fp8_rescaled(lo.y, s_prev, s), 0u);
  return enc_pair<true>(fp8_rescaled(hi.x, s_prev, s), fp8_rescaled(hi.y, s_prev, s), o);
}

}  // namespace pa
