// quantize.hip -- device packer: f32 or bf16 [n,k] in HBM -> codes + block scales.
//
// The same encoding as the host packer (pack_math.hpp: per-block scale from
// the block amax, codes against the stored scale, fp64 quotients), computed on
// the GPU so a weight never has to visit the host to be re-packed
// [rlx-cpu quant.rs, lowp_compute_scales and lowp_quantize, which the pages
// run as producer ops of the scaled matmul].
//
// MX formats (the activation formats of the scaled-MFMA GEMM): a lane owns 8
// consecutive elements, so one 32-block is a quad of lanes and every load is a
// coalesced 16- or 32-byte run.  The quad's amax (two lane swaps) gives the
// E8M0 byte; each element is then scaled by 2^(127-b) in f32, which is the
// exact quotient whenever the result is a normal f32 (results below 2^-126 lie
// under every format's smallest rounding threshold, so they encode to a signed
// zero either way), and rounded onto the minifloat grid by a power-of-two
// rescale and rintf (nearest, ties to even): the same codes as the fp64
// encoder, with no fp64 arithmetic.
//
// Other formats: one thread packs one block with the fp64 encoder (their
// scales are not powers of two, so the quotient needs the wider type).
// nvfp4 first reduces the tensor amax into the caller's device float (vector
// atomicMax on the bits of non-negative floats), then turns it into the
// global scale in place.
#include "bsq_internal.hpp"
#include "pack_math.hpp"

namespace bsq {
namespace {

__global__ void amax_init(float *g) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *g = 0.0f;
}

// Loads 8 consecutive inputs (f32 or bf16) as f32 values.
template <int XT>
__device__ __forceinline__ void load8(const void *base, int64_t idx, float x[8]) {
  if constexpr (XT == 0) {
    const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + idx);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    const uint4 v = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + idx);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(u[i] << 16);
      x[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
}

template <int XT>
__global__ void __launch_bounds__(256) amax_kernel(const void *__restrict__ w, int64_t n8, unsigned *__restrict__ g) {
  float a = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    float x[8];
    load8<XT>(w, i * 8, x);
#pragma unroll
    for (int q = 0; q < 8; ++q) a = fmaxf(a, fabsf(x[q]));
  }
  // wave-level max first: one atomic per wave
  for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
  if ((threadIdx.x & 63) == 0) atomicMax(g, __float_as_uint(a));
}

__global__ void global_finalize(float *g) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *g = pk::nvfp4_global(*g);
}

// Nearest-even code of a finite a >= 0 on a minifloat grid with M mantissa
// bits and exponent bias BT (subnormals included), clamped to MAXC.  a * 2^-qe
// is exact (a power-of-two rescale of an f32 that neither overflows nor
// underflows), so rintf decides the rounding exactly.
template <int M, int BT, int MAXC>
__device__ __forceinline__ uint32_t grid_code(float a) {
  if (!(a > 0.0f)) return 0u;
  int ex;
  frexpf(a, &ex);  // a in [2^(ex-1), 2^ex)
  const int e = ex - 1, emin = 1 - BT;
  const int qe = (e < emin ? emin : e) - M;
  const int q = (int)rintf(ldexpf(a, -qe));
  const int code = e < emin ? q : ((e + BT) << M) + q - (1 << M);
  return (uint32_t)(code < MAXC ? code : MAXC);
}

template <int F> struct MxEnc;
template <> struct MxEnc<kMXFP4> {
  static constexpr int kEmax = 2;
  __device__ static uint32_t enc(float v) { return grid_code<1, 1, 7>(fabsf(v)) | (signbit(v) ? 8u : 0u); }
};
template <> struct MxEnc<kMXFP8_E4M3> {
  static constexpr int kEmax = 8;
  __device__ static uint32_t enc(float v) { return grid_code<3, 7, 0x7E>(fabsf(v)) | (signbit(v) ? 0x80u : 0u); }
};
template <> struct MxEnc<kMXFP8_E5M2> {
  static constexpr int kEmax = 15;
  __device__ static uint32_t enc(float v) { return grid_code<2, 15, 0x7B>(fabsf(v)) | (signbit(v) ? 0x80u : 0u); }
};

template <int F, int XT>
__global__ void __launch_bounds__(256)
quantize_mx_kernel(const void *__restrict__ w, int64_t n8, uint8_t *__restrict__ codes,
                   uint8_t *__restrict__ scales, int *__restrict__ status) {
  // n8 (elements / 8) is a multiple of 4, so a quad is always wholly inside
  // or outside the range and the lane swaps read active lanes only.
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n8; t += (int64_t)gridDim.x * blockDim.x) {
    float x[8];
    load8<XT>(w, t * 8, x);
    float a = 0.0f;
    bool finite = true;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      finite = finite && isfinite(x[i]);
      a = fmaxf(a, fabsf(x[i]));
    }
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    if (!finite && status) *status = 5;  // BSQ_ERR_NONFINITE; the block's bytes are then unspecified
    int sb = 127;
    if (a > 0.0f) {
      int ex;
      frexpf(a, &ex);
      int e = ex - 1 - MxEnc<F>::kEmax;
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
      sb = e + 127;
    }
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = MxEnc<F>::enc(ldexpf(x[i], 127 - sb));
    if constexpr (F == kMXFP4) {
      uint32_t wd = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) wd |= c[i] << (4 * i);
      reinterpret_cast<uint32_t *>(codes)[t] = wd;
    } else {
      const uint32_t lo = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
      const uint32_t hi = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
      reinterpret_cast<uint2 *>(codes)[t] = make_uint2(lo, hi);
    }
    if ((t & 3) == 0) scales[t >> 2] = (uint8_t)sb;
  }
}

template <int F, int XT>
__global__ void __launch_bounds__(256)
quantize_kernel(const void *__restrict__ w, int64_t n, int64_t k, const float *__restrict__ gdev,
                uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, uint8_t *__restrict__ biases,
                int *__restrict__ status) {
  constexpr int B = Traits<F>::kBlock;
  const int64_t nb = k / B, blocks = n * nb;
  const float g = (F == kNVFP4) ? *gdev : 1.0f;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < blocks; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t j = t / nb, b = t - j * nb;
    float x[B];
#pragma unroll
    for (int i = 0; i < B; i += 8) load8<XT>(w, j * k + b * B + i, x + i);
    bool finite = true;
#pragma unroll
    for (int i = 0; i < B; ++i) finite = finite && isfinite(x[i]);
    if (!finite && status) *status = 5;  // BSQ_ERR_NONFINITE; the block's bytes are then unspecified
    uint8_t c[B];
    uint32_t sb, bb;
    pk::pack_block<F>(x, g, c, &sb, &bb);
    const int64_t p0 = j * k + b * B;
    if constexpr (Traits<F>::kBits == 4) {
      uint32_t words[B / 8];
#pragma unroll
      for (int q = 0; q < B / 8; ++q) {
        uint32_t wd = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) wd |= (uint32_t)(c[8 * q + i] & 0xF) << (4 * i);
        words[q] = wd;
      }
      uint32_t *dst = reinterpret_cast<uint32_t *>(codes + p0 / 2);
      if constexpr (B / 8 == 2) {
        *reinterpret_cast<uint2 *>(dst) = make_uint2(words[0], words[1]);
      } else {
#pragma unroll
        for (int q = 0; q < B / 8; q += 4)
          *reinterpret_cast<uint4 *>(dst + q) = make_uint4(words[q], words[q + 1], words[q + 2], words[q + 3]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < B; q += 16) {
        uint32_t wd[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          wd[r] = (uint32_t)c[q + 4 * r] | ((uint32_t)c[q + 4 * r + 1] << 8) | ((uint32_t)c[q + 4 * r + 2] << 16) |
                  ((uint32_t)c[q + 4 * r + 3] << 24);
        *reinterpret_cast<uint4 *>(codes + p0 + q) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
    }
    if constexpr (F == kNVFP8 || F == kINT8_SYM) {
      reinterpret_cast<uint32_t *>(scales)[t] = sb;
    } else if constexpr (F == kINT4_AFFINE) {
      reinterpret_cast<uint16_t *>(scales)[t] = (uint16_t)sb;
      reinterpret_cast<uint16_t *>(biases)[t] = (uint16_t)bb;
    } else {
      scales[t] = (uint8_t)sb;
    }
  }
}

template <int F, int XT>
hipError_t run(const void *w, int64_t n, int64_t k, void *codes, void *scales, void *biases, float *gdev,
               int *status, hipStream_t s) {
  if constexpr (F == kNVFP4) {
    hipLaunchKernelGGL(amax_init, dim3(1), dim3(64), 0, s, gdev);
    const int64_t n8 = n * k / 8;
    int64_t blocks = (n8 + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(amax_kernel<XT>, dim3((unsigned)blocks), dim3(256), 0, s, w, n8,
                       reinterpret_cast<unsigned *>(gdev));
    hipLaunchKernelGGL(global_finalize, dim3(1), dim3(64), 0, s, gdev);
  }
  if constexpr (F == kMXFP4 || F == kMXFP8_E4M3 || F == kMXFP8_E5M2) {
    const int64_t n8 = n * k / 8;
    int64_t grid = (n8 + 255) / 256;
    if (grid > 65536) grid = 65536;
    if (grid > 0)
      hipLaunchKernelGGL((quantize_mx_kernel<F, XT>), dim3((unsigned)grid), dim3(256), 0, s, w, n8, (uint8_t *)codes,
                         (uint8_t *)scales, status);
    return hipGetLastError();
  }
  const int64_t nblocks = n * (k / Traits<F>::kBlock);
  int64_t grid = (nblocks + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL((quantize_kernel<F, XT>), dim3((unsigned)grid), dim3(256), 0, s, w, n, k, gdev,
                     (uint8_t *)codes, (uint8_t *)scales, (uint8_t *)biases, status);
  return hipGetLastError();
}

template <int F>
hipError_t run_t(const void *w, int wt, int64_t n, int64_t k, void *codes, void *scales, void *biases, float *gdev,
                 int *status, hipStream_t s) {
  return wt == 1 ? run<F, 1>(w, n, k, codes, scales, biases, gdev, status, s)
                 : run<F, 0>(w, n, k, codes, scales, biases, gdev, status, s);
}

}  // namespace

hipError_t launch_quantize(int fmt, const void *w, int wt, int64_t n, int64_t k, void *codes, void *scales,
                           void *biases, float *gdev, int *status, hipStream_t s) {
  switch (fmt) {
    case kMXFP4: return run_t<kMXFP4>(w, wt, n, k, codes, scales, biases, gdev, status, s);
    case kNVFP4: return run_t<kNVFP4>(w, wt, n, k, codes, scales, biases, gdev, status, s);
    case kMXFP8_E4M3: return run_t<kMXFP8_E4M3>(w, wt, n, k, codes, scales, biases, gdev, status, s);
    case kMXFP8_E5M2: return run_t<kMXFP8_E5M2>(w, wt, n, k, codes, scales, biases, gdev, status, s);
    case kNVFP8: return run_t<kNVFP8>(w, wt, n, k, codes, scales, biases, gdev, status, s);
    case kINT4_AFFINE: return run_t<kINT4_AFFINE>(w, wt, n, k, codes, scales, biases, gdev, status, s);
    case kINT8_SYM: return run_t<kINT8_SYM>(w, wt, n, k, codes, scales, biases, gdev, status, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace bsq
