// pack_host.cpp -- host packer: f32 [n,k] -> codes + per-block scales.
//
// The encoding rule (pack_math.hpp) is shared with the device quantize
// kernel; rows are packed in parallel with std::thread.  Non-finite input is
// rejected before anything is written.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "bsq_internal.hpp"
#include "pack_math.hpp"

namespace bsq {
namespace {

// Packs rows [j0, j1) of w into the stored layout of format F.
template <int F>
void pack_rows(const float *w, int64_t k, float g, uint8_t *codes, uint8_t *scales, uint8_t *biases, int64_t j0,
               int64_t j1) {
  constexpr int B = Traits<F>::kBlock;
  const int64_t nb = k / B;
  uint8_t c[64];
  for (int64_t j = j0; j < j1; ++j) {
    for (int64_t b = 0; b < nb; ++b) {
      uint32_t sb, bb;
      pk::pack_block<F>(w + j * k + b * B, g, c, &sb, &bb);
      const int64_t si = j * nb + b, p0 = j * k + b * B;
      if constexpr (Traits<F>::kBits == 4) {
        for (int i = 0; i < B; i += 2) codes[(p0 + i) >> 1] = (uint8_t)((c[i] & 0xF) | ((c[i + 1] & 0xF) << 4));
      } else {
        std::memcpy(codes + p0, c, B);
      }
      if constexpr (F == kNVFP8 || F == kINT8_SYM) {
        std::memcpy(scales + 4 * si, &sb, 4);
      } else if constexpr (F == kINT4_AFFINE) {
        const uint16_t s16 = (uint16_t)sb, b16 = (uint16_t)bb;
        std::memcpy(scales + 2 * si, &s16, 2);
        std::memcpy(biases + 2 * si, &b16, 2);
      } else {
        scales[si] = (uint8_t)sb;
      }
    }
  }
}

template <int F>
void pack_all(const float *w, int64_t n, int64_t k, float g, uint8_t *codes, uint8_t *scales, uint8_t *biases) {
  const int64_t nt = std::max<int64_t>(1, std::min<int64_t>(std::thread::hardware_concurrency(), n / 64));
  if (nt <= 1) {
    pack_rows<F>(w, k, g, codes, scales, biases, 0, n);
    return;
  }
  std::vector<std::thread> th;
  const int64_t per = (n + nt - 1) / nt;
  for (int64_t t = 0; t < nt; ++t) {
    const int64_t j0 = std::min(n, t * per), j1 = std::min(n, j0 + per);
    th.emplace_back([=] { pack_rows<F>(w, k, g, codes, scales, biases, j0, j1); });
  }
  for (auto &x : th) x.join();
}

}  // namespace

int pack_host(int fmt, const float *w, int64_t n, int64_t k, void *codes, void *scales, void *biases,
              float *global_out) {
  for (int64_t i = 0; i < n * k; ++i)
    if (!std::isfinite(w[i])) return 5;  // BSQ_ERR_NONFINITE
  float g = 1.0f;
  if (fmt == kNVFP4) {
    float T = 0.0f;
    for (int64_t i = 0; i < n * k; ++i) T = std::max(T, std::fabs(w[i]));
    g = pk::nvfp4_global(T);
  }
  if (global_out) *global_out = g;
  uint8_t *c = (uint8_t *)codes, *s = (uint8_t *)scales, *b = (uint8_t *)biases;
  switch (fmt) {
    case kMXFP4: pack_all<kMXFP4>(w, n, k, g, c, s, b); break;
    case kNVFP4: pack_all<kNVFP4>(w, n, k, g, c, s, b); break;
    case kMXFP8_E4M3: pack_all<kMXFP8_E4M3>(w, n, k, g, c, s, b); break;
    case kMXFP8_E5M2: pack_all<kMXFP8_E5M2>(w, n, k, g, c, s, b); break;
    case kNVFP8: pack_all<kNVFP8>(w, n, k, g, c, s, b); break;
    case kINT4_AFFINE: pack_all<kINT4_AFFINE>(w, n, k, g, c, s, b); break;
    case kINT8_SYM: pack_all<kINT8_SYM>(w, n, k, g, c, s, b); break;
    default: return 2;
  }
  return 0;
}

}  // namespace bsq
