// rows.hip -- VALU streaming kernel for f32 activations (any m, routed or not), the fused
// RMSNorm beyond the one-row bf16 case, and bf16 rows the decode GEMV kernel
// (gemv.hip) does not take (stacks of 2 GiB of codes or more):
// out[i,j] = sum_p X[i,p] * dequant(W)[j,p].
//
// The weight stream is the cost ("the win is memory bandwidth, not flops,
// since LLM weights dominate the working set" [rlx-cpu quant.rs,
// dequant_matmul_int8]), so each weight row is read from HBM once per launch
// with 16-byte loads and decoded in registers; every X row of the launch's
// m-chunk reuses the decoded codes.
//
// Geometry (gfx950, wave64): a wave owns RPW weight rows at a time.  Lane l
// takes 16-byte code chunks l, l+64, l+128, ... along k (32 elements for 4-bit
// codes, 16 for 8-bit).  The code, scale and X loads of a round (U chunks of
// all RPW rows) are issued back to back before any arithmetic; full rounds
// carry no bounds checks, so no wait separates them.  Per 8-element sub-chunk
// the
// unscaled element values are dotted with X in fp32; the block scale is folded
// once per block, not per element [rlx-cpu quant.rs, dequant_matmul_int8,
// which applies each block's scale a single time] and the nvfp4 global once at the end
// [rlx-cpu quant.rs, dequant_matmul_nvfp4].  int4 affine folds s and b per
// group as s * sum(q*x) + b * sum(x) [metaltile-std tests/qmm_gpu_correctness.rs,
// cpu_qmm_reference].  The wave's partial sums are reduced with DPP row
// permutes and two cross-row swaps.
//
// bf16 X uses the gfx950 conversions (v_cvt_scalef32_pk_bf16_fp4/fp8/bf8 with
// scale 1.0, which are exact for these element sets) and v_dot2_f32_bf16; f32
// X uses the gfx950 f32 conversions (v_cvt_scalef32_pk_f32_fp4/fp8/bf8) and
// fp32 FMA; the integer formats use branch-free software decoders.
//
// Fused RMSNorm (NORM): the activation is x * g / sqrt(mean(x^2) + eps) per
// row [metaltile PR #250, commit adding the block-scaled fused RMSNorm +
// dequantizing GEMV: sum x^2 into the row's inverse RMS, then the GEMV over
// x * norm_weight * inv_rms].  The inverse RMS is one factor per row, so it
// comes out of the sum: each wave, which streams the whole row of x anyway,
// accumulates sum x^2 alongside its dot products over x * g (in f32, for
// either x dtype) and scales its outputs once at the end; no extra pass.
//
// Expert routing (eids != null, one X row per launch row): X row i multiplies
// expert eids[i] of a stacked [E*n, k] weight, i.e. weight rows eids[i]*n ..
// eids[i]*n + n - 1 [metaltile PR #250, commit adding the per-token
// expert-routed qmm: one indirection, the stack kept as one packed tensor so
// nvfp4's single global stays valid].  An id outside [0, E) loads nothing,
// leaves that output row zero and sets *status to 1 (BSQ_ERR_ARG).
#include "bsq_internal.hpp"
#include "codec.hpp"
#include "dot.hpp"

#include <type_traits>

namespace bsq {
namespace {

using namespace dot;

constexpr int kWaves = 4;  // waves per workgroup

// A wave owns RPW consecutive weight rows.  A round covers U 16-byte code
// chunks per lane of each row.  Full rounds (every chunk inside k) are
// branch-free: all code, scale (and, when it fits in registers, X) loads of
// the round are issued before any arithmetic, so each wave keeps RPW*U HBM
// requests in flight with no wait between them.  A ragged last round runs
// the same code with bounds guards.  XLN (fused RMSNorm, one bf16 x row,
// k <= kXlnMax): the workgroup first forms x*g in f32 in LDS and the row's
// sum of squares once, so the rounds load only codes and scales (measured:
// 4096^2 nvfp4 6.15 -> 5.9 us; the norm weight loads, one per x load, were
// the fused kernel's extra cost).
constexpr int kXlnMax = 8192;
template <int F, int M, int XT, bool VEC, int RPW, int U, bool NORM, bool XLN = false>
__global__ void __launch_bounds__(kWaves * 64)
rows_kernel(const uint8_t *__restrict__ codes, const void *__restrict__ scales, const uint16_t *__restrict__ biases,
            float global, const void *__restrict__ xv, void *__restrict__ out, int ot, int64_t m, int64_t n, int64_t k,
            const void *__restrict__ gam, float eps, const int32_t *__restrict__ eids, int64_t nexp,
            int *__restrict__ status) {
  constexpr int B = Traits<F>::kBlock;
  constexpr int E = Traits<F>::kBits == 4 ? 32 : 16;  // elements per 16-byte chunk
  constexpr int NSUB = E / 8;                           // 8-element sub-chunks per chunk
  constexpr int NB = B < E ? E / B : 1;                 // scale blocks per chunk
  constexpr int SPB = NSUB / NB;                        // sub-chunks per scale block
  constexpr int XW = XT == 1 ? 1 : 2;                   // uint4 per 8 X values
  constexpr bool XPRE = M * U * NSUB * XW <= 16;        // X of a round fits in 64 VGPRs
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  const int64_t i0 = (int64_t)blockIdx.y * M;  // first X row of this launch chunk
  const int64_t nblk = k / B;
  const int64_t row_bytes = Traits<F>::kBits == 4 ? k / 2 : k;
  const int64_t per_round = (int64_t)64 * E * U;
  const int64_t full_rounds = VEC ? k / per_round : 0;
  static_assert(!XLN || (NORM && M == 1 && XT == 1 && VEC), "LDS x*g: fused RMSNorm, one bf16 row");
  int64_t xrow[M];
#pragma unroll
  for (int mi = 0; mi < M; ++mi) xrow[mi] = (i0 + mi < m ? i0 + mi : m - 1) * k;  // rows past m: valid, unused
  // expert routing: first weight row of this X row's expert (M == 1 here)
  int64_t jbase = 0;
  bool skip = false;
  if (eids) {
    const int64_t e = eids[i0];
    skip = e < 0 || e >= nexp;
    if (skip && status && blockIdx.x == 0 && threadIdx.x == 0) *status = 1;
    jbase = skip ? 0 : e * n;
  }

  __shared__ __attribute__((aligned(16))) float xg[XLN ? kXlnMax : 4];
  __shared__ float redw[XLN ? kWaves : 1];
  float xln_rinv = 1.0f;
  if constexpr (XLN) {
    // x*g (exact in f32: a product of two bf16) into LDS, and sum x^2 over the row
    const uint16_t *xr = reinterpret_cast<const uint16_t *>(xv) + xrow[0];
    float ss = 0.0f;
    for (int64_t p = (int64_t)threadIdx.x * 8; p < k; p += kWaves * 64 * 8) {
      const uint4 a = *reinterpret_cast<const uint4 *>(xr + p);
      const uint4 gv = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(gam) + p);
      const uint32_t xs4[4] = {a.x, a.y, a.z, a.w}, gs4[4] = {gv.x, gv.y, gv.z, gv.w};
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = __uint_as_float(xs4[i] << 16), x1 = __uint_as_float(xs4[i] & 0xFFFF0000u);
        ss = __builtin_fmaf(x0, x0, ss);
        ss = __builtin_fmaf(x1, x1, ss);
        f[2 * i] = x0 * __uint_as_float(gs4[i] << 16);
        f[2 * i + 1] = x1 * __uint_as_float(gs4[i] & 0xFFFF0000u);
      }
      *reinterpret_cast<float4 *>(&xg[p]) = make_float4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<float4 *>(&xg[p + 4]) = make_float4(f[4], f[5], f[6], f[7]);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) redw[threadIdx.x >> 6] = ss;
    __syncthreads();
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += redw[w];
    xln_rinv = 1.0f / sqrtf(t / (float)k + eps);
  }

  for (int64_t j0 = wave * RPW; j0 < n; j0 += nwaves * RPW) {
    float acc[RPW][M], ssq[M];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int mi = 0; mi < M; ++mi) acc[r][mi] = 0.0f;
#pragma unroll
    for (int mi = 0; mi < M; ++mi) ssq[mi] = 0.0f;
    int64_t jr[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) jr[r] = jbase + (j0 + r < n ? j0 + r : n - 1);  // rows past n: valid, never stored

    auto round = [&](auto guard, int64_t kc0) {
      constexpr bool kG = decltype(guard)::value;
      // ---- phase A: the round's loads ----
      uint4 cw[RPW][U];
      uint32_t sr[RPW][U][NB], br[RPW][U];
      uint4 xq[XPRE ? M : 1][XPRE ? U : 1][XPRE ? NSUB * XW : 1];
      uint4 gq[NORM && XPRE ? U : 1][NORM && XPRE ? NSUB * XW : 1];  // norm gain of the round
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const uint8_t *crow = codes + jr[r] * row_bytes;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t kc = kc0 + (int64_t)u * 64 * E;
          const int64_t off = Traits<F>::kBits == 4 ? kc / 2 : kc;
          if (!kG) {
            // bf16 X (decode and m <= 8: one X chunk per launch) reads each
            // weight byte once: a streaming (nontemporal) load, measured 5-8%
            // faster on the decode shapes; f32 X chunks re-read the rows
            if constexpr (XT == 1) {
              const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(crow + off));
              cw[r][u] = make_uint4(t.x, t.y, t.z, t.w);
            } else {
              cw[r][u] = *reinterpret_cast<const uint4 *>(crow + off);
            }
          } else {
            uint32_t t[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (kc + (int64_t)(q + 1) * E / 4 <= k) t[q] = reinterpret_cast<const uint32_t *>(crow + off)[q];
            cw[r][u] = make_uint4(t[0], t[1], t[2], t[3]);
          }
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const int64_t pb = kc + (int64_t)b * (E / NB);
            const int64_t bi = (!kG || pb < k) ? pb / B : nblk - 1;
            sr[r][u][b] = load_scale_raw<F>(scales, jr[r] * nblk + bi);
          }
          if constexpr (F == kINT4_AFFINE) br[r][u] = biases[jr[r] * nblk + ((!kG || kc < k) ? kc / B : nblk - 1)];
        }
      }
      if constexpr (XPRE && !XLN) {
#pragma unroll
        for (int mi = 0; mi < M; ++mi)
#pragma unroll
          for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < NSUB * XW; ++q) {
              const int64_t p = kc0 + (int64_t)u * 64 * E + (q / XW) * 8;
              if (!kG || p < k) {
                if constexpr (XT == 1)
                  xq[mi][u][q] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(xv) + xrow[mi] + p);
                else
                  xq[mi][u][q] = reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(xv) + xrow[mi] + p)[q % XW];
              } else {
                xq[mi][u][q] = make_uint4(0, 0, 0, 0);
              }
            }
        if constexpr (NORM) {
#pragma unroll
          for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < NSUB * XW; ++q) {
              const int64_t p = kc0 + (int64_t)u * 64 * E + (q / XW) * 8;
              if (!kG || p < k) {
                if constexpr (XT == 1)
                  gq[u][q] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(gam) + p);
                else
                  gq[u][q] = reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(gam) + p)[q % XW];
              } else {
                gq[u][q] = make_uint4(0, 0, 0, 0);
              }
            }
        }
      }
      // keep every load of the round ahead of the arithmetic
      __builtin_amdgcn_sched_barrier(0);
      // ---- phase B: decode, dot, fold ----
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t kc = kc0 + (int64_t)u * 64 * E;
        if (kG && kc >= k) break;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int64_t pb = kc + (int64_t)b * (E / NB);
          if (kG && pb >= k) break;
          float part[RPW][M], xsum[M];
#pragma unroll
          for (int mi = 0; mi < M; ++mi) {
            xsum[mi] = 0.0f;
#pragma unroll
            for (int r = 0; r < RPW; ++r) part[r][mi] = 0.0f;
          }
#pragma unroll
          for (int s = b * SPB; s < (b + 1) * SPB; ++s) {
            const int64_t p = kc + 8 * s;
            if (kG && p >= k) break;
#pragma unroll
            for (int mi = 0; mi < M; ++mi) {
              if (i0 + mi >= m) break;
              uint4 xa, xb2;
              if constexpr (XLN) {
                xa = xb2 = make_uint4(0, 0, 0, 0);  // x*g comes from LDS below
              } else if constexpr (XPRE) {
                xa = xq[mi][u][s * XW];
                xb2 = xq[mi][u][s * XW + XW - 1];
              } else if constexpr (XT == 1) {
                xa = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(xv) + xrow[mi] + p);
                xb2 = xa;
              } else {
                const uint4 *xp = reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(xv) + xrow[mi] + p);
                xa = xp[0];
                xb2 = xp[1];
              }
              if constexpr (NORM) {
                // x as f32, its squares into the row's sum, then x * g
                float xf[8], gf[8];
                if constexpr (XLN) {
                  const float4 a = *reinterpret_cast<const float4 *>(&xg[p]);
                  const float4 b = *reinterpret_cast<const float4 *>(&xg[p + 4]);
                  xf[0] = a.x, xf[1] = a.y, xf[2] = a.z, xf[3] = a.w, xf[4] = b.x, xf[5] = b.y, xf[6] = b.z, xf[7] = b.w;
#pragma unroll
                  for (int i = 0; i < 8; ++i) gf[i] = 1.0f;
                } else if constexpr (XT == 1) {
                  const uint32_t xs[4] = {xa.x, xa.y, xa.z, xa.w};
                  uint4 gv;
                  if constexpr (XPRE) gv = gq[u][s * XW];
                  else gv = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(gam) + p);
                  const uint32_t gs[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    xf[2 * i] = __uint_as_float(xs[i] << 16);
                    xf[2 * i + 1] = __uint_as_float(xs[i] & 0xFFFF0000u);
                    gf[2 * i] = __uint_as_float(gs[i] << 16);
                    gf[2 * i + 1] = __uint_as_float(gs[i] & 0xFFFF0000u);
                  }
                } else {
                  uint4 ga, gb;
                  if constexpr (XPRE) {
                    ga = gq[u][s * XW];
                    gb = gq[u][s * XW + XW - 1];
                  } else {
                    const uint4 *gp = reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(gam) + p);
                    ga = gp[0];
                    gb = gp[1];
                  }
                  const uint32_t xs[8] = {xa.x, xa.y, xa.z, xa.w, xb2.x, xb2.y, xb2.z, xb2.w};
                  const uint32_t gs[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
#pragma unroll
                  for (int i = 0; i < 8; ++i) {
                    xf[i] = __uint_as_float(xs[i]);
                    gf[i] = __uint_as_float(gs[i]);
                  }
                }
                if constexpr (!XLN) {
#pragma unroll
                  for (int i = 0; i < 8; ++i) {
                    ssq[mi] = __builtin_fmaf(xf[i], xf[i], ssq[mi]);
                    xf[i] *= gf[i];
                  }
                }
#pragma unroll
                for (int r = 0; r < RPW; ++r) {
                  const uint32_t cwa[4] = {cw[r][u].x, cw[r][u].y, cw[r][u].z, cw[r][u].w};
                  const uint32_t w0 = Traits<F>::kBits == 4 ? cwa[s] : cwa[2 * s];
                  const uint32_t w1 = Traits<F>::kBits == 4 ? 0u : cwa[2 * s + 1];
                  part[r][mi] = dot8_f32<F>(w0, w1, xf, part[r][mi]);
                }
                if constexpr (F == kINT4_AFFINE)
                  xsum[mi] += ((xf[0] + xf[1]) + (xf[2] + xf[3])) + ((xf[4] + xf[5]) + (xf[6] + xf[7]));
                continue;
              }
#pragma unroll
              for (int r = 0; r < RPW; ++r) {
                const uint32_t cwa[4] = {cw[r][u].x, cw[r][u].y, cw[r][u].z, cw[r][u].w};
                const uint32_t w0 = Traits<F>::kBits == 4 ? cwa[s] : cwa[2 * s];
                const uint32_t w1 = Traits<F>::kBits == 4 ? 0u : cwa[2 * s + 1];
                if constexpr (XT == 1) {
                  part[r][mi] = dot8_bf16<F>(w0, w1, xa, part[r][mi]);
                } else {
                  const float xf[8] = {__uint_as_float(xa.x), __uint_as_float(xa.y), __uint_as_float(xa.z),
                                       __uint_as_float(xa.w), __uint_as_float(xb2.x), __uint_as_float(xb2.y),
                                       __uint_as_float(xb2.z), __uint_as_float(xb2.w)};
                  part[r][mi] = dot8_f32<F>(w0, w1, xf, part[r][mi]);
                }
              }
              if constexpr (F == kINT4_AFFINE) {
                if constexpr (XT == 1) {
                  const uint32_t xs[4] = {xa.x, xa.y, xa.z, xa.w};
#pragma unroll
                  for (int i = 0; i < 4; ++i)
                    xsum[mi] += __uint_as_float(xs[i] << 16) + __uint_as_float(xs[i] & 0xFFFF0000u);
                } else {
                  xsum[mi] += ((__uint_as_float(xa.x) + __uint_as_float(xa.y)) + (__uint_as_float(xa.z) + __uint_as_float(xa.w))) +
                              ((__uint_as_float(xb2.x) + __uint_as_float(xb2.y)) + (__uint_as_float(xb2.z) + __uint_as_float(xb2.w)));
                }
              }
            }
          }
#pragma unroll
          for (int r = 0; r < RPW; ++r) {
            const float sc = scale_value<F>(sr[r][u][b]);
#pragma unroll
            for (int mi = 0; mi < M; ++mi) {
              acc[r][mi] = __builtin_fmaf(part[r][mi], sc, acc[r][mi]);
              if constexpr (F == kINT4_AFFINE) acc[r][mi] = __builtin_fmaf(xsum[mi], bf16_bits_to_f32(br[r][u]), acc[r][mi]);
            }
          }
        }
      }
    };

    const int64_t lane0 = (int64_t)lane * E;
    if (!skip) {
      for (int64_t rr = 0; rr < full_rounds; ++rr) round(std::integral_constant<bool, false>{}, lane0 + rr * per_round);
      // guarded rounds to the end of k: one ragged round when VEC, every round
      // when the code rows are not 16-byte aligned (then full_rounds == 0)
      for (int64_t base = full_rounds * per_round; base < k; base += per_round)
        round(std::integral_constant<bool, true>{}, lane0 + base);
    }

    float rinv[M];
#pragma unroll
    for (int mi = 0; mi < M; ++mi)
      rinv[mi] = NORM ? (XLN ? xln_rinv : 1.0f / sqrtf(wave_sum(ssq[mi]) / (float)k + eps)) : 1.0f;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
#pragma unroll
      for (int mi = 0; mi < M; ++mi) {
        float v = wave_sum(acc[r][mi]);
        if constexpr (F == kNVFP4) v *= global;
        if constexpr (NORM) v *= rinv[mi];
        if (lane == r * M + mi && j0 + r < n && i0 + mi < m) {
          const int64_t o = (i0 + mi) * n + j0 + r;
          if (ot == 0) reinterpret_cast<float *>(out)[o] = v;
          else reinterpret_cast<uint16_t *>(out)[o] = f32_to_bf16_bits(v);
        }
      }
    }
  }
}

// Routing arguments of a launch (eids == nullptr: no routing).
struct Route {
  const int32_t *eids;
  int64_t nexp;
  int *status;
};

template <int F, int M, int XT, int RPW, int U, bool NORM>
hipError_t run_cfg(const QWeight &w, int64_t m, const void *x, void *out, int ot, const void *gam, float eps,
                   const Route &rt, hipStream_t s) {
  const bool vec = Traits<F>::kBits == 8 || (w.k % 32) == 0;  // 16-byte aligned code rows
  const int64_t waves = (w.n + RPW - 1) / RPW;
  int64_t wgs = (waves + kWaves - 1) / kWaves;
  if (wgs > 8192) wgs = 8192;
  const int64_t ychunks = (m + M - 1) / M;
  const dim3 grid((unsigned)wgs, (unsigned)ychunks);
  constexpr bool kXlnCfg = NORM && M == 1 && XT == 1;
  if (kXlnCfg && vec && w.k <= kXlnMax)
    hipLaunchKernelGGL((rows_kernel<F, M, XT, true, RPW, U, NORM, kXlnCfg>), grid, dim3(kWaves * 64), 0, s,
                       (const uint8_t *)w.codes, w.scales, (const uint16_t *)w.biases, w.global, x, out, ot, m, w.n,
                       w.k, gam, eps, rt.eids, rt.nexp, rt.status);
  else if (vec)
    hipLaunchKernelGGL((rows_kernel<F, M, XT, true, RPW, U, NORM>), grid, dim3(kWaves * 64), 0, s,
                       (const uint8_t *)w.codes, w.scales, (const uint16_t *)w.biases, w.global, x, out, ot, m, w.n,
                       w.k, gam, eps, rt.eids, rt.nexp, rt.status);
  else if constexpr (!NORM)  // the fused RMSNorm requires whole 16-byte code rows (checked by the caller)
    hipLaunchKernelGGL((rows_kernel<F, M, XT, false, RPW, U, false>), grid, dim3(kWaves * 64), 0, s,
                       (const uint8_t *)w.codes, w.scales, (const uint16_t *)w.biases, w.global, x, out, ot, m, w.n,
                       w.k, gam, eps, rt.eids, rt.nexp, rt.status);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Rows per wave and chunks per round: the bf16 decode GEMV (M <= 2) keeps
// two rows' code loads in flight per wave, one chunk per row and round for
// 4-bit codes and two for 8-bit codes (measured best on the 4096x4096 nvfp4
// and 14336x4096 mxfp8 decode shapes); wider M reuses each decoded chunk M
// times and keeps one row per wave to bound registers.
template <int F, int M, int XT, bool NORM>
hipError_t run_m(const QWeight &w, int64_t m, const void *x, void *out, int ot, const void *gam, float eps,
                 const Route &rt, hipStream_t s) {
  constexpr int U = Traits<F>::kBits == 4 ? 1 : 2;  // 16-byte chunks per row per round
  if constexpr (M <= 2 && XT == 1) return run_cfg<F, M, XT, 2, U, NORM>(w, m, x, out, ot, gam, eps, rt, s);
  else return run_cfg<F, M, XT, 1, 2, NORM>(w, m, x, out, ot, gam, eps, rt, s);
}

template <int F, int XT, bool NORM>
hipError_t run_x(const QWeight &w, int64_t m, const void *x, void *out, int ot, const void *gam, float eps,
                 const Route &rt, hipStream_t s) {
  if (m <= 1 || rt.eids) return run_m<F, 1, XT, NORM>(w, m, x, out, ot, gam, eps, rt, s);  // routed: a row each
  if (m <= 2) return run_m<F, 2, XT, NORM>(w, m, x, out, ot, gam, eps, rt, s);
  if (m <= 4) return run_m<F, 4, XT, NORM>(w, m, x, out, ot, gam, eps, rt, s);
  return run_m<F, 8, XT, NORM>(w, m, x, out, ot, gam, eps, rt, s);
}

template <int F, bool NORM>
hipError_t run_f(const QWeight &w, int64_t m, const void *x, int xt, void *out, int ot, const void *gam, float eps,
                 const Route &rt, hipStream_t s) {
  if (m > (rt.eids ? (int64_t)65535 : (int64_t)65535 * 8)) return hipErrorInvalidValue;
  return xt == 1 ? run_x<F, 1, NORM>(w, m, x, out, ot, gam, eps, rt, s)
                 : run_x<F, 0, NORM>(w, m, x, out, ot, gam, eps, rt, s);
}

template <bool NORM>
hipError_t launch(const QWeight &w, int64_t m, const void *x, int xt, void *out, int ot, const void *gam, float eps,
                  const Route &rt, hipStream_t s) {
  switch (w.fmt) {
    case kMXFP4: return run_f<kMXFP4, NORM>(w, m, x, xt, out, ot, gam, eps, rt, s);
    case kNVFP4: return run_f<kNVFP4, NORM>(w, m, x, xt, out, ot, gam, eps, rt, s);
    case kMXFP8_E4M3: return run_f<kMXFP8_E4M3, NORM>(w, m, x, xt, out, ot, gam, eps, rt, s);
    case kMXFP8_E5M2: return run_f<kMXFP8_E5M2, NORM>(w, m, x, xt, out, ot, gam, eps, rt, s);
    case kNVFP8: return run_f<kNVFP8, NORM>(w, m, x, xt, out, ot, gam, eps, rt, s);
    case kINT4_AFFINE: return run_f<kINT4_AFFINE, NORM>(w, m, x, xt, out, ot, gam, eps, rt, s);
    case kINT8_SYM: return run_f<kINT8_SYM, NORM>(w, m, x, xt, out, ot, gam, eps, rt, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_rows(const QWeight &w, int64_t m, const void *x, int xt, void *out, int ot, hipStream_t s) {
  // one bf16 activation row: the decode GEMV kernel (gemv.hip)
  if (gemv_applies(w, m, xt, false)) return launch_gemv(w, m, x, out, ot, nullptr, 0, nullptr, s);
  // a few bf16 rows: its multi-row form, one weight pass per 4 rows (gemv.hip)
  if (xt == 1 && m <= kGemvDenseRows && gemv_grouped_applies(w, m, 1))
    return launch_gemv_grouped(w, m, 1, nullptr, x, out, ot, nullptr, s);
  return launch<false>(w, m, x, xt, out, ot, nullptr, 0.0f, Route{nullptr, 0, nullptr}, s);
}

hipError_t launch_rows_norm(const QWeight &w, int64_t m, const void *x, int xt, const void *gam, float eps, void *out,
                            int ot, hipStream_t s) {
  return launch<true>(w, m, x, xt, out, ot, gam, eps, Route{nullptr, 0, nullptr}, s);
}

hipError_t launch_rows_gather(const QWeight &w, int64_t m, const void *x, int xt, const int32_t *eids, int64_t nexp,
                              int *status, void *out, int ot, hipStream_t s) {
  if (gemv_applies(w, m, xt, true)) return launch_gemv(w, m, x, out, ot, eids, nexp, status, s);
  return launch<false>(w, m, x, xt, out, ot, nullptr, 0.0f, Route{eids, nexp, status}, s);
}

}  // namespace bsq
