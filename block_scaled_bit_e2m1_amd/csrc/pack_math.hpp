// pack_math.hpp -- the library's encoders and per-block packing rule, shared
// by the host packer (pack_host.cpp) and the device quantize kernel
// (quantize.hip), so the two produce identical bytes.
//
// Scale choice per block along k, then every element encoded against the
// scale as stored (the "effective" scale), so codes and scales are
// self-consistent [metaltile PR #250, commit "QFormat {Nvfp4, Mxfp4, Mxfp8E4,
// Mxfp8E5, Nvfp8} with pack() and dequant()"; rlx-cpu quant.rs,
// lowp_compute_scales and lowp_quantize].
//
// Element encoders:
//   E2M1 by comparing with the midpoints between levels, a tie going to
//        the even-mantissa code;
//   E4M3 / E5M2 / bf16 by integer rounding of the fp64 significand (nearest,
//        ties to even), saturating E4M3 at +-448 (the format has no inf)
//        and finite E5M2 inputs at +-57344
//   [metaltile PR #250, codec commits].
// Quotients w / S are formed in fp64, which decides every rounding exactly
// for these operand widths.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bsq_internal.hpp"

namespace bsq {
namespace pk {

#define BSQ_HD __host__ __device__ __forceinline__

// Nearest-even rounding of a >= 0 onto a minifloat with `mbits` mantissa bits
// and exponent bias `bias` (subnormals included); returns the magnitude code
// (exponent field << mbits | mantissa), clamped to `max_code`.
BSQ_HD uint32_t minifloat_code(double a, int mbits, int bias, uint32_t max_code) {
  if (!(a > 0.0)) return 0;
  int ex;
  const double f = frexp(a, &ex);                    // a = f * 2^ex, f in [0.5, 1)
  const uint64_t sig = (uint64_t)ldexp(f, 53);      // a = sig * 2^(ex-53), exact
  const int e = ex - 1;                              // a in [2^e, 2^(e+1))
  const int emin = 1 - bias;
  const int quantum_exp = (e < emin ? emin : e) - mbits;  // grid spacing 2^quantum_exp
  const int shift = quantum_exp - (ex - 53);               // bits of sig below the grid
  uint64_t q;
  if (shift >= 60) {
    q = 0;
  } else {
    q = sig >> shift;
    const uint64_t rem = sig & ((1ull << shift) - 1), half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
  }
  int64_t code;
  if (e < emin) {
    code = (int64_t)q;  // subnormal field; q == 2^mbits carries into exponent 1
  } else {
    code = ((int64_t)(e + bias) << mbits) + (int64_t)q - (1ll << mbits);
  }
  if (code > (int64_t)max_code) code = max_code;
  return (uint32_t)code;
}

BSQ_HD uint32_t sign_bit(double v, uint32_t bit) { return signbit(v) ? bit : 0u; }

// E2M1: the seven midpoints between consecutive levels
// {0,.5,1,1.5,2,3,4,6}; at a midpoint the even code wins.
BSQ_HD uint32_t enc_e2m1(double v) {
  const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  const double a = fabs(v);
  uint32_t c = 0;
  for (int i = 0; i < 7; ++i) {
    const uint32_t up = (uint32_t)i + 1;
    if (a > mid[i] || (a == mid[i] && (up & 1u) == 0)) c = up;
  }
  return c | sign_bit(v, 8u);
}
BSQ_HD uint32_t enc_e4m3(double v) { return minifloat_code(fabs(v), 3, 7, 0x7E) | sign_bit(v, 0x80u); }
BSQ_HD uint32_t enc_e5m2(double v) { return minifloat_code(fabs(v), 2, 15, 0x7B) | sign_bit(v, 0x80u); }
BSQ_HD uint16_t enc_bf16(double v) {
  const uint32_t c = minifloat_code(fabs(v), 7, 127, 0x7F80);  // 0x7F80 = inf
  return (uint16_t)(c | sign_bit(v, 0x8000u));
}

BSQ_HD double e4m3_value(uint32_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  const double mag = e ? ldexp(8.0 + m, e - 10) : ldexp((double)m, -9);
  return (c & 0x80) ? -mag : mag;
}
BSQ_HD double bf16_value(uint16_t h) {
  union {
    uint32_t u;
    float f;
  } x;
  x.u = (uint32_t)h << 16;
  return x.f;
}

// E8M0 byte for a block: floor(log2(amax)) minus the element's top exponent,
// clamped to [-127, 127]; 127 (scale 1) for an all-zero block.
BSQ_HD uint32_t e8m0_for(double amax, int elem_emax) {
  if (amax == 0.0) return 127;
  int ex;
  frexp(amax, &ex);
  int e = ex - 1 - elem_emax;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  return (uint32_t)(e + 127);
}

// nvfp4 global scale from the tensor amax: f32(T / (6 * 448)), 1 if that is 0.
BSQ_HD float nvfp4_global(float T) {
  const float g = T / 2688.0f;
  return (g > 0.0f) ? g : 1.0f;
}

// Packs one block of B = block_of(fmt) consecutive weights x[0..B).
// code[i] receives the code of element i (a nibble or a byte); *scale_bits
// the stored scale (u8 code, f32 bits or bf16 bits); *bias_bits the int4 bias.
// g is the nvfp4 global (ignored otherwise).
template <int F>
BSQ_HD void pack_block(const float *x, float g, uint8_t *code, uint32_t *scale_bits, uint32_t *bias_bits) {
  constexpr int B = Traits<F>::kBlock;
  double amax = 0.0, lo = x[0], hi = x[0];
  for (int i = 0; i < B; ++i) {
    const double a = fabs((double)x[i]);
    amax = a > amax ? a : amax;
    lo = (double)x[i] < lo ? (double)x[i] : lo;
    hi = (double)x[i] > hi ? (double)x[i] : hi;
  }
  *bias_bits = 0;
  if constexpr (F == kMXFP4 || F == kMXFP8_E4M3 || F == kMXFP8_E5M2) {
    const int emax = F == kMXFP4 ? 2 : (F == kMXFP8_E4M3 ? 8 : 15);
    const uint32_t sb = e8m0_for(amax, emax);
    *scale_bits = sb;
    const double S = ldexp(1.0, (int)sb - 127);
    for (int i = 0; i < B; ++i) {
      const double v = x[i] / S;
      code[i] = (uint8_t)(F == kMXFP4 ? enc_e2m1(v) : (F == kMXFP8_E4M3 ? enc_e4m3(v) : enc_e5m2(v)));
    }
  } else if constexpr (F == kNVFP4) {
    const uint32_t micro = amax == 0.0 ? 0x38u : enc_e4m3(amax / (6.0 * (double)g));
    *scale_bits = micro;
    const double S = e4m3_value(micro) * (double)g;
    for (int i = 0; i < B; ++i) code[i] = (uint8_t)(S != 0.0 ? enc_e2m1(x[i] / S) : 0u);
  } else if constexpr (F == kNVFP8 || F == kINT8_SYM) {
    const float s = amax == 0.0 ? 1.0f : (float)amax / (F == kNVFP8 ? 448.0f : 127.0f);
    union {
      float f;
      uint32_t u;
    } sv;
    sv.f = s;
    *scale_bits = sv.u;
    const double S = s;
    for (int i = 0; i < B; ++i) {
      uint32_t c = 0;
      if (S != 0.0) {
        if constexpr (F == kNVFP8) {
          c = enc_e4m3(x[i] / S);
        } else {
          double q = rint(x[i] / S);
          q = q > 127.0 ? 127.0 : (q < -127.0 ? -127.0 : q);
          c = (uint32_t)(uint8_t)(int8_t)q;
        }
      }
      code[i] = (uint8_t)c;
    }
  } else {  // int4 affine
    const uint16_t sb = enc_bf16((hi - lo) / 15.0), bb = enc_bf16(lo);
    *scale_bits = sb;
    *bias_bits = bb;
    const double s = bf16_value(sb), bias = bf16_value(bb);
    for (int i = 0; i < B; ++i) {
      double q = 0.0;
      if (s != 0.0) {
        q = rint(((double)x[i] - bias) / s);
        q = q > 15.0 ? 15.0 : (q < 0.0 ? 0.0 : q);
      }
      code[i] = (uint8_t)q;
    }
  }
}

#undef BSQ_HD

}  // namespace pk
}  // namespace bsq
