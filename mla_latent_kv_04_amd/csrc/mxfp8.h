// MXFP8 latent-cache row format and the gfx950 conversions that encode and
// decode it.
//
// The pages cache the latent at four bits (NVFP4) and gather it with 16-byte
// loads ("撕开 DeepSeek MLA 源码", sheratonhq.com, section 5) without giving
// the code or the scale layout.  This library's format is the CDNA4-native
// analogue: OCP MXFP8 -- E4M3 codes (bias 7, no infinities, largest 448) in
// blocks of 32 consecutive latent values that share one E8M0 scale byte
// s (value 2^(s - 127)).  A block's scale is the smallest power of two 2^X with
// max |v| <= 448 * 2^X (no element saturates), X clamped to [-127, 127]; an
// all-zero block takes s = 0.  Codes are v / 2^X rounded to nearest, ties to
// even.  The k_R branch stays bf16.
//
// Row of one token (656 bytes, each part 16-byte aligned):
//   [0, 512)    latent codes, one byte each
//   [512, 528)  the 16 scale bytes, block j covering latent values 32j .. 32j+31
//   [528, 656)  k_R, 64 bf16
// A page is 64 rows (41 984 bytes); paging is the bf16 cache's.
#pragma once

#include "common.h"

namespace mla {

constexpr int kF8Codes = 0;
constexpr int kF8Scales = kLatent;                    // 512
constexpr int kF8Rope = kF8Scales + kLatent / 32;     // 528
constexpr int kF8RowBytes = kF8Rope + kRope * 2;      // 656
constexpr int kF8PageBytes = kPage * kF8RowBytes;     // 41984

typedef short s16x2 __attribute__((ext_vector_type(2)));

// E8M0 scale byte of a block from its largest magnitude (finite, >= 0): X + 127 for
// the smallest X with amax <= 448 * 2^X.  With amax = 1.m * 2^(e - 127), X is
// e - 135 (amax / 2^X in [256, 512)), one more when 1.m > 1.75.
__device__ __forceinline__ int mx_scale_byte(float amax) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, amax);
  const int e = (int)(bits >> 23) & 0xFF;
  if (e == 0) return 0;                                 // zero or below 2^-126: X clamps to -127
  const int x = e - 135 + ((bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  const int s = x + 127;
  return s < 0 ? 0 : (s > 254 ? 254 : s);
}

// Two values already divided by their block scale (|v| <= 448) -> E4M3 codes in the
// low (kHi = false) or high 16 bits of `old`; round to nearest, ties to even.
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3_pack2(uint32_t old, float a, float b) {
  const s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(s16x2, old), a, b, 1.0f, kHi);
  return __builtin_bit_cast(uint32_t, r);
}

// Four codes (one dword) -> four bf16 (two dwords) times the block scale 2^(s - 127):
// exact for normal bf16 results.  The conversion uses only the exponent field of
// the fp32 scale operand, which is the scale byte itself.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(uint32_t codes, float scale) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, scale, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, scale, true);
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

__device__ __forceinline__ float mx_scale_f32(uint32_t scale_byte) {
  return __builtin_bit_cast(float, scale_byte << 23);
}

}  // namespace mla
