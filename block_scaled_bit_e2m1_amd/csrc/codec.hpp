// codec.hpp -- branch-free device decoders for the block-scaled formats.
//
// Every decoder returns the exact f32 value of its code; the only rounding in
// a dequantized weight is the one f32 multiply by the block scale.
//
// Formats [metaltile PR #250, commit "Foundation for the spec-conformant
// nvfp4/mxfp4/mxfp8/nvfp8 formats"; metaltile-std src/mlx/fp_quantized_mma.rs,
// module doc sections "fp4 E2M1 codebook" and "fp8 E4M3 dequant"]:
//   E2M1  [s:1][e:2][m:1], levels {0, .5, 1, 1.5, 2, 3, 4, 6}
//   E4M3  [s:1][e:4][m:3], bias 7, saturating variant: only S.1111.111 is NaN
//   E5M2  the high byte of an IEEE binary16
//   E8M0  2^(b-127); b = 255 is NaN
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace bsq {

// E2M1 magnitude: twice each of the eight levels is an integer < 16, so the
// whole codebook fits the nibbles of one 32-bit immediate (nibble i = 2*level
// of code i).  No shift by a negative amount, no branch.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t twice = (0xC8643210u >> ((c & 7u) << 2)) & 0xFu;
  const float mag = (float)twice * 0.5f;
  return __uint_as_float(__float_as_uint(mag) | ((c & 8u) << 28));
}

// E4M3: placing the 7 magnitude bits at f32 bit 20 makes an f32 whose
// exponent field is the E4M3 exponent field and whose top mantissa bits are
// the E4M3 mantissa; scaling by 2^(127-7) rebiases it.  For the subnormal
// codes the same placement is an f32 subnormal m * 2^-129, and the product is
// m * 2^-9, so one multiply covers both cases exactly (f32 denormals kept).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t em = c & 0x7Fu;
  float mag = __uint_as_float(em << 20) * 0x1p120f;
  mag = (em == 0x7Fu) ? __uint_as_float(0x7FC00000u) : mag;
  return __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
}

// E5M2: exactly the binary16 whose high byte is the code.
__device__ __forceinline__ float e5m2_to_f32(uint32_t c) {
  return __half2float(__ushort_as_half((unsigned short)((c & 0xFFu) << 8)));
}

// E8M0 scale 2^(b-127): b << 23 is that power of two for b in [1,254]; b = 0
// is the f32 subnormal 2^-127 (bit 22); b = 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  b &= 0xFFu;
  const uint32_t bits = (b == 0u) ? 0x00400000u : (b == 255u ? 0x7FC00000u : (b << 23));
  return __uint_as_float(bits);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float((h & 0xFFFFu) << 16); }

// f32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

}  // namespace bsq
