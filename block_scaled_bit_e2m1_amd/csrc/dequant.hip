// dequant.hip -- standalone dequant: codes + scales -> f32 [n,k].
//
// One thread per 8 consecutive elements (one u32 of 4-bit codes or 8 bytes
// of 8-bit codes), written as two 16-byte stores.  An elementwise kernel with
// a bounds guard, no reduction [metaltile PR #250, "First spec-conformant
// block-scaled dequant kernel: mt_mxfp4_dequant" and the commit completing the
// standalone dequant kernels].  Each value is decode(code) * scale with a
// single f32 rounding (nvfp4: (e2m1 * e4m3) * global, the first product
// exact; int4: fma(s, q, b)), so the result is bit-identical to the exact
// value rounded once to f32.
#include "bsq_internal.hpp"
#include "codec.hpp"

namespace bsq {
namespace {

template <int F>
__device__ __forceinline__ float elem_value(uint32_t c) {
  if constexpr (F == kMXFP4 || F == kNVFP4) return e2m1_to_f32(c);
  else if constexpr (F == kMXFP8_E4M3 || F == kNVFP8) return e4m3_to_f32(c);
  else if constexpr (F == kMXFP8_E5M2) return e5m2_to_f32(c);
  else if constexpr (F == kINT4_AFFINE) return (float)(c & 0xFu);
  else return (float)(int8_t)(uint8_t)c;
}

template <int F>
__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t *__restrict__ codes, const void *__restrict__ scales,
                                                      const uint16_t *__restrict__ biases, float global,
                                                      float *__restrict__ out, int64_t n, int64_t k) {
  constexpr int B = Traits<F>::kBlock;
  const int64_t chunks = n * k / 8;
  const int64_t nblk = k / B;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < chunks; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e0 = t * 8;
    const int64_t j = e0 / k, p0 = e0 - j * k;
    const int64_t si = j * nblk + p0 / B;  // 8 elements never straddle a block (8 | B)
    uint32_t cw[8];
    if constexpr (Traits<F>::kBits == 4) {
      const uint32_t word = reinterpret_cast<const uint32_t *>(codes)[t];
#pragma unroll
      for (int i = 0; i < 8; ++i) cw[i] = (word >> (4 * i)) & 0xFu;
    } else {
      const uint2 v = reinterpret_cast<const uint2 *>(codes)[t];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        cw[i] = (v.x >> (8 * i)) & 0xFFu;
        cw[4 + i] = (v.y >> (8 * i)) & 0xFFu;
      }
    }
    float r[8];
    if constexpr (F == kMXFP4 || F == kMXFP8_E4M3 || F == kMXFP8_E5M2) {
      const float s = e8m0_to_f32(reinterpret_cast<const uint8_t *>(scales)[si]);
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = elem_value<F>(cw[i]) * s;
    } else if constexpr (F == kNVFP4) {
      const float s = e4m3_to_f32(reinterpret_cast<const uint8_t *>(scales)[si]);
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = (elem_value<F>(cw[i]) * s) * global;
    } else if constexpr (F == kNVFP8 || F == kINT8_SYM) {
      const float s = reinterpret_cast<const float *>(scales)[si];
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = elem_value<F>(cw[i]) * s;
    } else {
      const float s = bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(scales)[si]);
      const float b = bf16_bits_to_f32(biases[si]);
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = __builtin_fmaf(s, elem_value<F>(cw[i]), b);
    }
    float4 *o = reinterpret_cast<float4 *>(out + e0);
    o[0] = make_float4(r[0], r[1], r[2], r[3]);
    o[1] = make_float4(r[4], r[5], r[6], r[7]);
  }
}

__global__ void zero_kernel(uint8_t *__restrict__ out, int64_t bytes) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < bytes; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = 0;
}

template <int F>
hipError_t run(const QWeight &w, float *out, hipStream_t s) {
  const int64_t chunks = w.n * w.k / 8;
  const int64_t blocks = (chunks + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(dequant_kernel<F>, dim3(grid), dim3(256), 0, s, (const uint8_t *)w.codes, w.scales,
                     (const uint16_t *)w.biases, w.global, out, w.n, w.k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(const QWeight &w, float *out, hipStream_t s) {
  switch (w.fmt) {
    case kMXFP4: return run<kMXFP4>(w, out, s);
    case kNVFP4: return run<kNVFP4>(w, out, s);
    case kMXFP8_E4M3: return run<kMXFP8_E4M3>(w, out, s);
    case kMXFP8_E5M2: return run<kMXFP8_E5M2>(w, out, s);
    case kNVFP8: return run<kNVFP8>(w, out, s);
    case kINT4_AFFINE: return run<kINT4_AFFINE>(w, out, s);
    case kINT8_SYM: return run<kINT8_SYM>(w, out, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_zero(void *out, int64_t bytes, hipStream_t s) {
  const int64_t blocks = (bytes + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s, (uint8_t *)out, bytes);
  return hipGetLastError();
}

}  // namespace bsq
