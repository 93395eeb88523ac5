// pack_host.cpp -- host packer: f32 [n,k] -> codes + per-block scales.
//
// Scale choice per block along k, then every element encoded against the
// scale as stored (the "effective" scale), so codes and scales are
// self-consistent [metaltile PR #250, commit "QFormat {Nvfp4, Mxfp4, Mxfp8E4,
// Mxfp8E5, Nvfp8} with pack() and dequant()"; rlx-cpu quant.rs,
// lowp_compute_scales and lowp_quantize].
//
// Element encoders:
//   E2M1 by midpoint thresholds ("midpoint-threshold encode"), a tie going to
//        the even-mantissa code;
//   E4M3 / E5M2 / bf16 by integer rounding of the fp64 significand (nearest,
//        ties to even), saturating E4M3 at 448 ("+-448 saturation, no inf")
//        and E5M2 at 57344 ("e5m2_encode now saturates finite inputs")
//   [metaltile PR #250, codec commits].
// Quotients w / S are formed in fp64, which decides every rounding exactly
// for these operand widths.  Rows are packed in parallel (std::thread).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "bsq_internal.hpp"

namespace bsq {
namespace {

// Nearest-even rounding of |v| onto a minifloat with `mbits` mantissa bits and
// exponent bias `bias` (subnormals included); returns the magnitude code
// (exponent field << mbits | mantissa), clamped to `max_code`.
uint32_t minifloat_code(double a, int mbits, int bias, uint32_t max_code) {
  if (!(a > 0.0)) return 0;
  int ex;
  const double f = std::frexp(a, &ex);  // a = f * 2^ex, f in [0.5, 1)
  const uint64_t sig = (uint64_t)std::ldexp(f, 53);  // a = sig * 2^(ex-53), exact
  const int e = ex - 1;                               // a in [2^e, 2^(e+1))
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

inline uint32_t sign_bit(double v, uint32_t bit) { return std::signbit(v) ? bit : 0u; }

// E2M1: the seven midpoints between consecutive levels
// {0,.5,1,1.5,2,3,4,6}; at a midpoint the even code wins.
uint32_t enc_e2m1(double v) {
  static const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  const double a = std::fabs(v);
  uint32_t c = 0;
  for (int i = 0; i < 7; ++i) {
    const uint32_t up = (uint32_t)i + 1;
    if (a > mid[i] || (a == mid[i] && (up & 1u) == 0)) c = up;
  }
  return c | sign_bit(v, 8u);
}
uint32_t enc_e4m3(double v) { return minifloat_code(std::fabs(v), 3, 7, 0x7E) | sign_bit(v, 0x80u); }
uint32_t enc_e5m2(double v) { return minifloat_code(std::fabs(v), 2, 15, 0x7B) | sign_bit(v, 0x80u); }
uint16_t enc_bf16(double v) {
  uint32_t c = minifloat_code(std::fabs(v), 7, 127, 0x7F80);  // 0x7F80 = inf
  return (uint16_t)(c | sign_bit(v, 0x8000u));
}

double e4m3_value(uint32_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  const double mag = e ? std::ldexp(8.0 + m, e - 10) : std::ldexp((double)m, -9);
  return (c & 0x80) ? -mag : mag;
}
double bf16_value(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// E8M0 byte for a block: floor(log2(amax)) minus the element's top exponent,
// clamped to [-127, 127]; 127 (scale 1) for an all-zero block.
uint32_t e8m0_for(double amax, int elem_emax) {
  if (amax == 0.0) return 127;
  int ex;
  std::frexp(amax, &ex);
  int e = ex - 1 - elem_emax;
  e = std::min(127, std::max(-127, e));
  return (uint32_t)(e + 127);
}

struct Packer {
  int fmt, B;
  int64_t k;
  float g;
  uint8_t *codes;
  uint8_t *scales;
  uint8_t *biases;

  void put(int64_t j, int64_t p, uint32_t c) const {
    if (is_4bit(fmt)) {
      uint8_t &byte = codes[(j * k + p) >> 1];
      if (p & 1)
        byte = (uint8_t)((byte & 0x0F) | ((c & 0xF) << 4));
      else
        byte = (uint8_t)((byte & 0xF0) | (c & 0xF));
    } else {
      codes[j * k + p] = (uint8_t)c;
    }
  }

  void row(const float *w, int64_t j) const {
    const int64_t nb = k / B;
    for (int64_t b = 0; b < nb; ++b) {
      const float *x = w + j * k + b * B;
      const int64_t p0 = b * B, si = j * nb + b;
      double amax = 0.0, lo = x[0], hi = x[0];
      for (int i = 0; i < B; ++i) {
        amax = std::max(amax, std::fabs((double)x[i]));
        lo = std::min(lo, (double)x[i]);
        hi = std::max(hi, (double)x[i]);
      }
      switch (fmt) {
        case kMXFP4: case kMXFP8_E4M3: case kMXFP8_E5M2: {
          const int emax = fmt == kMXFP4 ? 2 : (fmt == kMXFP8_E4M3 ? 8 : 15);
          const uint32_t sb = e8m0_for(amax, emax);
          scales[si] = (uint8_t)sb;
          const double S = std::ldexp(1.0, (int)sb - 127);
          for (int i = 0; i < B; ++i) {
            const double v = x[i] / S;
            put(j, p0 + i, fmt == kMXFP4 ? enc_e2m1(v) : (fmt == kMXFP8_E4M3 ? enc_e4m3(v) : enc_e5m2(v)));
          }
          break;
        }
        case kNVFP4: {
          const uint32_t micro = amax == 0.0 ? 0x38u : enc_e4m3(amax / (6.0 * (double)g));
          scales[si] = (uint8_t)micro;
          const double S = e4m3_value(micro) * (double)g;
          for (int i = 0; i < B; ++i) put(j, p0 + i, S != 0.0 ? enc_e2m1(x[i] / S) : 0u);
          break;
        }
        case kNVFP8: case kINT8_SYM: {
          const float s = amax == 0.0 ? 1.0f : (float)amax / (fmt == kNVFP8 ? 448.0f : 127.0f);
          std::memcpy(scales + 4 * si, &s, 4);
          const double S = s;
          for (int i = 0; i < B; ++i) {
            uint32_t c = 0;
            if (S != 0.0) {
              if (fmt == kNVFP8) {
                c = enc_e4m3(x[i] / S);
              } else {
                const double q = std::min(127.0, std::max(-127.0, std::nearbyint(x[i] / S)));
                c = (uint32_t)(uint8_t)(int8_t)q;
              }
            }
            put(j, p0 + i, c);
          }
          break;
        }
        case kINT4_AFFINE: {
          const uint16_t sb = enc_bf16((hi - lo) / 15.0), bb = enc_bf16(lo);
          std::memcpy(scales + 2 * si, &sb, 2);
          std::memcpy(biases + 2 * si, &bb, 2);
          const double s = bf16_value(sb), bias = bf16_value(bb);
          for (int i = 0; i < B; ++i) {
            double q = 0.0;
            if (s != 0.0) q = std::min(15.0, std::max(0.0, std::nearbyint(((double)x[i] - bias) / s)));
            put(j, p0 + i, (uint32_t)q);
          }
          break;
        }
      }
    }
  }
};

}  // namespace

int pack_host(int fmt, const float *w, int64_t n, int64_t k, void *codes, void *scales, void *biases,
              float *global_out) {
  const int B = block_of(fmt);
  for (int64_t i = 0; i < n * k; ++i)
    if (!std::isfinite(w[i])) return 5;  // BSQ_ERR_NONFINITE
  float g = 1.0f;
  if (fmt == kNVFP4) {
    float T = 0.0f;
    for (int64_t i = 0; i < n * k; ++i) T = std::max(T, std::fabs(w[i]));
    g = T / 2688.0f;  // 6 * 448: the largest E2M1 level times the largest E4M3 value
    if (!(g > 0.0f)) g = 1.0f;
  }
  if (global_out) *global_out = g;
  if (is_4bit(fmt)) std::memset(codes, 0, (size_t)(n * k / 2));
  Packer P{fmt, B, k, g, (uint8_t *)codes, (uint8_t *)scales, (uint8_t *)biases};
  const int64_t nt = std::max<int64_t>(1, std::min<int64_t>(std::thread::hardware_concurrency(), n / 64));
  if (nt <= 1) {
    for (int64_t j = 0; j < n; ++j) P.row(w, j);
  } else {
    std::vector<std::thread> th;
    for (int64_t t = 0; t < nt; ++t)
      th.emplace_back([&, t] {
        for (int64_t j = t; j < n; j += nt) P.row(w, j);
      });
    for (auto &x : th) x.join();
  }
  return 0;
}

}  // namespace bsq
