// calib.hip -- the two measurements that give the roofline denominators as
// this device reaches them, next to the vendor figures:
//  * a streaming read of a device buffer with the decode kernel's load form
//    (16-byte nontemporal vector loads, every byte read once, nothing
//    computed), the bandwidth ceiling a weight-streaming kernel can reach at
//    that size;
//  * a register-only loop of v_mfma_f32_32x32x16_bf16 (no memory traffic),
//    the bf16 matrix-core ceiling.
// Neither touches the hot path; both keep their loads / products alive with a
// data-dependent store that never fires for ordinary data.
#include "bsq_internal.hpp"

namespace bsq {
namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr uint32_t kNever = 0x9E3779B9u;  // a sum of loaded words this equals is not stored for real data

__global__ void __launch_bounds__(256) read_kernel(const v4u *__restrict__ p, int64_t nchunks, float *__restrict__ sink) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nchunks) return;
  const v4u v = __builtin_nontemporal_load(p + i);
  if ((v.x ^ v.y ^ v.z ^ v.w) == kNever) sink[0] = 1.0f;
}

// Each wave: `iters` steps of four independent 32x32x16 bf16 MFMAs.
__global__ void __launch_bounds__(256) mfma_loop_kernel(int64_t iters, float *__restrict__ sink) {
  const uint32_t l = threadIdx.x;
  const uint4 u = make_uint4(0x3F803F80u ^ l, 0x3F803F80u, 0x3F803F80u ^ (l << 3), 0x3F803F80u);
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, u);
  f32x16_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = (float)(c + v);
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[c], 0, 0, 0);
  }
  float t = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) t += acc[c][0] + acc[c][15];
  if (__float_as_uint(t) == kNever) sink[0] = t;
}

}  // namespace

hipError_t launch_calib_read(const void *buf, int64_t bytes, float *sink, hipStream_t s) {
  const int64_t nchunks = bytes / 16;
  const int64_t wgs = (nchunks + 255) / 256;
  if (wgs == 0) return hipSuccess;
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)wgs), dim3(256), 0, s, (const v4u *)buf, nchunks, sink);
  return hipGetLastError();
}

hipError_t launch_calib_mfma(int64_t iters, int64_t workgroups, float *sink, hipStream_t s) {
  if (workgroups <= 0 || workgroups > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)workgroups), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace bsq
