// dot.hpp -- per-element decode and 8-element dot products shared by the
// streaming kernels (rows.hip, gemv.hip), and the wave-level sum.
//
// bf16 x: the gfx950 conversions v_cvt_scalef32_pk_bf16_{fp4,fp8,bf8} with
// scale 1.0 (exact: every E2M1, E4M3 and E5M2 value is a bf16) feed
// v_dot2_f32_bf16; the integer formats use branch-free software decoders and
// fp32 FMA.  f32 x: the f32 conversions and fp32 FMA.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsq_internal.hpp"
#include "codec.hpp"

namespace bsq {
namespace dot {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

// Sum over the 64 lanes of a wave; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // half-row mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row mirror
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Unscaled element values of one 8-element sub-chunk: the gfx950 f32
// conversions for the minifloat elements (scale 1.0: exact, since every E2M1,
// E4M3 and E5M2 value is an f32), software decoders for the integers.
template <int F>
__device__ __forceinline__ void decode8(uint32_t w0, uint32_t w1, float e[8]) {
  typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
  if constexpr (F == kMXFP4 || F == kNVFP4) {
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w0, 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w0, 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w0, 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w0, 1.0f, 3);
    e[0] = p0[0]; e[1] = p0[1]; e[2] = p1[0]; e[3] = p1[1];
    e[4] = p2[0]; e[5] = p2[1]; e[6] = p3[0]; e[7] = p3[1];
  } else if constexpr (F == kMXFP8_E4M3 || F == kNVFP8) {
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w0, 1.0f, false);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w0, 1.0f, true);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w1, 1.0f, false);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w1, 1.0f, true);
    e[0] = p0[0]; e[1] = p0[1]; e[2] = p1[0]; e[3] = p1[1];
    e[4] = p2[0]; e[5] = p2[1]; e[6] = p3[0]; e[7] = p3[1];
  } else if constexpr (F == kMXFP8_E5M2) {
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(w0, 1.0f, false);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(w0, 1.0f, true);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(w1, 1.0f, false);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(w1, 1.0f, true);
    e[0] = p0[0]; e[1] = p0[1]; e[2] = p1[0]; e[3] = p1[1];
    e[4] = p2[0]; e[5] = p2[1]; e[6] = p3[0]; e[7] = p3[1];
  } else if constexpr (Traits<F>::kBits == 4) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = (w0 >> (4 * i)) & 0xFu;
      if constexpr (F == kINT4_AFFINE) e[i] = (float)c;
      else e[i] = e2m1_to_f32(c);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = ((i < 4 ? w0 : w1) >> (8 * (i & 3))) & 0xFFu;
      if constexpr (F == kMXFP8_E4M3 || F == kNVFP8) e[i] = e4m3_to_f32(c);
      else if constexpr (F == kMXFP8_E5M2) e[i] = e5m2_to_f32(c);
      else e[i] = (float)(int8_t)(uint8_t)c;
    }
  }
}

// acc + sum_i elem_i * x_i for 8 elements with bf16 x (packed pairs in xv).
template <int F>
__device__ __forceinline__ float dot8_bf16(uint32_t w0, uint32_t w1, uint4 xv, float acc) {
  if constexpr (F == kMXFP4 || F == kNVFP4) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w0, 1.0f, 0), as_bf16x2(xv.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w0, 1.0f, 1), as_bf16x2(xv.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w0, 1.0f, 2), as_bf16x2(xv.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w0, 1.0f, 3), as_bf16x2(xv.w), acc, false);
    return acc;
  } else if constexpr (F == kMXFP8_E4M3 || F == kNVFP8) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false), as_bf16x2(xv.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true), as_bf16x2(xv.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false), as_bf16x2(xv.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true), as_bf16x2(xv.w), acc, false);
    return acc;
  } else if constexpr (F == kMXFP8_E5M2) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, 1.0f, false), as_bf16x2(xv.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, 1.0f, true), as_bf16x2(xv.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, 1.0f, false), as_bf16x2(xv.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, 1.0f, true), as_bf16x2(xv.w), acc, false);
    return acc;
  } else {
    float e[8];
    decode8<F>(w0, w1, e);
    const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = __builtin_fmaf(e[2 * i], __uint_as_float(xs[i] << 16), acc);
      acc = __builtin_fmaf(e[2 * i + 1], __uint_as_float(xs[i] & 0xFFFF0000u), acc);
    }
    return acc;
  }
}

template <int F>
__device__ __forceinline__ float dot8_f32(uint32_t w0, uint32_t w1, const float x[8], float acc) {
  float e[8];
  decode8<F>(w0, w1, e);
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(e[i], x[i], acc);
  return acc;
}

// Raw scale word of row j, block b (decoded after all loads are in flight).
template <int F>
__device__ __forceinline__ uint32_t load_scale_raw(const void *scales, int64_t idx) {
  if constexpr (F == kMXFP4 || F == kMXFP8_E4M3 || F == kMXFP8_E5M2 || F == kNVFP4)
    return reinterpret_cast<const uint8_t *>(scales)[idx];
  else if constexpr (F == kNVFP8 || F == kINT8_SYM) return reinterpret_cast<const uint32_t *>(scales)[idx];
  else return reinterpret_cast<const uint16_t *>(scales)[idx];
}

template <int F>
__device__ __forceinline__ float scale_value(uint32_t raw) {
  if constexpr (F == kMXFP4 || F == kMXFP8_E4M3 || F == kMXFP8_E5M2) return e8m0_to_f32(raw);
  else if constexpr (F == kNVFP4) return e4m3_to_f32(raw);
  else if constexpr (F == kNVFP8 || F == kINT8_SYM) return __uint_as_float(raw);
  else return bf16_bits_to_f32(raw);
}

}  // namespace dot
}  // namespace bsq
