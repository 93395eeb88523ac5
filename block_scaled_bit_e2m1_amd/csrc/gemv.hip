// gemv.hip -- decode GEMV for bf16 activation rows that each stream the
// weight once: out[i,j] = sum_p x[i,p] * dequant(W)[j,p] for m = 1 (the
// decode step) and for every routed row of the expert gather.
//
// The weight stream is the whole cost of this step [rlx-cpu quant.rs,
// dequant_matmul_int8: memory bandwidth, not flops, since the weights dominate;
// metaltile PR #250, qgemv bench commit: the one-row-per-threadgroup kernels
// read latency-bound at low bandwidth].  Two measured facts about MI355X
// shape the design:
//  * A wave's 16-byte row loads spread over many HBM channels, so when every
//    wave issues all its loads at once each wave's data completes near the
//    end of the stream; the decode arithmetic (one VALU instruction per
//    element: v_cvt_scalef32_pk_bf16_* + v_dot2_f32_bf16, both full rate)
//    then runs after the data, not beside it.  Giving each wave several
//    row groups whose loads are consumed in issue order lets the first
//    groups' arithmetic overlap the rest of the stream.
//  * Per-row wave reductions cost about as much as the dot products at this
//    size, so the R rows of a group are reduced jointly: gfx950's
//    v_permlane32_swap / v_permlane16_swap fold 2 or 4 rows' partial sums
//    into halves / quarters of the wave, then 4 DPP steps finish all rows.
//
// Geometry: a workgroup of WPG waves; KW consecutive waves split the k
// chunks of a row group (lane l of wave ks takes the 16-byte chunk
// 64*(KW*round + ks) + l, i.e. 32 elements of 4-bit or 16 of 8-bit codes)
// and combine through LDS; each row group has S sequential groups of R rows.
// Loads are issued in the order the arithmetic consumes them, the first row
// group's codes ahead of everything else (x, the chunk's activations shared by
// all rows, follows them).  The block
// scale is folded once per block [rlx-cpu quant.rs, dequant_matmul_int8
// applies each block scale a single time], the nvfp4 global once at the end
// [rlx-cpu quant.rs, dequant_matmul_nvfp4], int4 as s*sum(q*x) + b*sum(x)
// [metaltile-std tests/qmm_gpu_correctness.rs, cpu_qmm_reference].
//
// Expert routing (eids != null): activation row i multiplies expert eids[i]
// of a stacked [E*n, k] weight [metaltile PR #250, commit adding the
// per-token expert-routed qmm]; an id outside [0, E) loads nothing, leaves
// that output row zero and sets *status to 1.
#include "bsq_internal.hpp"
#include "codec.hpp"
#include "dot.hpp"

#include <algorithm>
#include <type_traits>

namespace bsq {
namespace {

using namespace dot;

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Sum over each row of 16 lanes (every lane of the row receives it).
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // half-row mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row mirror
  return v;
}

// v_permlane32_swap: lanes 32..63 of a trade places with lanes 0..31 of b.
// Returns the sums lo + hi of the swapped pair: lanes 0..31 then hold
// a[l] + a[l+32], lanes 32..63 hold b[l-32] + b[l].
__device__ __forceinline__ float fold32(float a, float b) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// v_permlane16_swap: the same within each half, between 16-lane rows.
// Lanes 0..15 then hold a[l] + a[l+16], lanes 16..31 b[l-16] + b[l], and
// likewise for lanes 32..63.
__device__ __forceinline__ float fold16(float a, float b) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Joint wave reduction of R per-lane partial sums (R = 1, 2 or 4): row r's
// total lands in lane out_lane<R>(r).
template <int R>
__device__ __forceinline__ float joint_sum(const float (&a)[R]) {
  static_assert(R == 1 || R == 2 || R == 4, "joint reduction of 1, 2 or 4 rows");
  if constexpr (R == 1) {
    return wave_sum(a[0]);
  } else if constexpr (R == 2) {
    const float t = fold32(a[0], a[1]);  // lanes 0-31 row 0, 32-63 row 1
    return row16_sum(fold16(t, t));      // each 16-lane row: its half's total
  } else {
    const float s0 = fold32(a[0], a[2]);  // lanes 0-31 row 0, 32-63 row 2
    const float s1 = fold32(a[1], a[3]);  // lanes 0-31 row 1, 32-63 row 3
    return row16_sum(fold16(s0, s1));     // lanes 16r..16r+15: row r
  }
}
template <int R> __device__ __forceinline__ int out_lane(int r) { return R == 1 ? 0 : (R == 2 ? 32 * r : 16 * r); }

template <int F> constexpr int kE = Traits<F>::kBits == 4 ? 32 : 16;  // elements per 16-byte chunk
// chunks per stored scale word (nvfp4: one 16-bit pair of micro-scales per chunk)
template <int F> constexpr int kCPS = F == kNVFP4 ? 1 : (Traits<F>::kBlock > kE<F> ? Traits<F>::kBlock / kE<F> : 1);

// Raw scale (and int4 bias) of chunk ch of a row whose scales start at srow
// (bytes) and biases at brow.
template <int F>
__device__ __forceinline__ void load_sc(const uint8_t *__restrict__ srow, const uint16_t *__restrict__ brow,
                                        uint32_t ch, uint32_t &s, uint32_t &b) {
  if constexpr (F == kNVFP4) {
    s = *reinterpret_cast<const uint16_t *>(srow + 2 * ch);
  } else {
    const uint32_t bi = ch / kCPS<F>;
    s = load_scale_raw<F>(srow, bi);
    if constexpr (F == kINT4_AFFINE) b = brow[bi];
  }
}

// The block scale as f32.  E8M0: the hardware fp8 conversion of 1.0 with the
// byte as its exponent-only scale operand is exactly 2^(b-127), byte 0 giving
// the f32 subnormal 2^-127 and byte 255 NaN, with no compare.
template <int F>
__device__ __forceinline__ float block_scale(uint32_t s) {
  if constexpr (F == kMXFP4 || F == kMXFP8_E4M3 || F == kMXFP8_E5M2) {
    const f32x2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(0x38u, __uint_as_float((s & 0xFFu) << 23), false);
    return v[0];
  } else {
    return scale_value<F>(s);
  }
}

// acc + this chunk's contribution, its block scale(s) folded once.
template <int F>
__device__ __forceinline__ float chunk_dot(v4u c, uint32_t s, uint32_t b, const uint4 (&xq)[kE<F> / 8], float acc) {
  if constexpr (F == kNVFP4) {
    float p0 = dot8_bf16<F>(c.x, 0u, xq[0], 0.0f);
    p0 = dot8_bf16<F>(c.y, 0u, xq[1], p0);
    float p1 = dot8_bf16<F>(c.z, 0u, xq[2], 0.0f);
    p1 = dot8_bf16<F>(c.w, 0u, xq[3], p1);
    // both E4M3 micro-scales in one conversion (OCP E4M3: exact, 0x7F is NaN)
    const f32x2_t sv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s, 1.0f, false);
    acc = __builtin_fmaf(p0, sv[0], acc);
    return __builtin_fmaf(p1, sv[1], acc);
  } else if constexpr (F == kINT4_AFFINE) {
    // Each nibble pair becomes the exact bf16 pair (128 + q_even, 128 + q_odd)
    // (exponent 2^7, the nibble in the low mantissa bits): one byte permute
    // and an OR, then v_dot2 against x; 128 * sum(x) comes off afterwards,
    // sum(x) itself (for the bias) being v_dot2 against ones.
    const uint32_t wv[4] = {c.x, c.y, c.z, c.w};
    float p = 0.0f, xs = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t lo = wv[u] & 0x0F0F0F0Fu, hi = (wv[u] >> 4) & 0x0F0F0F0Fu;
      const uint32_t xv[4] = {xq[u].x, xq[u].y, xq[u].z, xq[u].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t pr =
            __builtin_amdgcn_perm(hi, lo, (0x0Cu << 24) | ((4u + t) << 16) | (0x0Cu << 8) | (uint32_t)t) | 0x43004300u;
        p = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pr), as_bf16x2(xv[t]), p, false);
        xs = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(0x3F803F80u), as_bf16x2(xv[t]), xs, false);
      }
    }
    acc = __builtin_fmaf(__builtin_fmaf(-128.0f, xs, p), block_scale<F>(s), acc);
    return __builtin_fmaf(xs, bf16_bits_to_f32(b), acc);
  } else if constexpr (Traits<F>::kBits == 4) {  // mxfp4: one scale per chunk
    float p = dot8_bf16<F>(c.x, 0u, xq[0], 0.0f);
    p = dot8_bf16<F>(c.y, 0u, xq[1], p);
    p = dot8_bf16<F>(c.z, 0u, xq[2], p);
    p = dot8_bf16<F>(c.w, 0u, xq[3], p);
    return __builtin_fmaf(p, block_scale<F>(s), acc);
  } else {  // 8-bit codes: 16 elements, one scale
    float p = dot8_bf16<F>(c.x, c.y, xq[0], 0.0f);
    p = dot8_bf16<F>(c.z, c.w, xq[1], p);
    return __builtin_fmaf(p, block_scale<F>(s), acc);
  }
}

// chunk_dot against f32 activations (the fused RMSNorm's x * g, exact in f32).
template <int F>
__device__ __forceinline__ float chunk_dot_f32(v4u c, uint32_t s, uint32_t b, const float (&xf)[kE<F>], float acc) {
  if constexpr (F == kNVFP4) {
    float p0 = dot8_f32<F>(c.x, 0u, xf + 0, 0.0f);
    p0 = dot8_f32<F>(c.y, 0u, xf + 8, p0);
    float p1 = dot8_f32<F>(c.z, 0u, xf + 16, 0.0f);
    p1 = dot8_f32<F>(c.w, 0u, xf + 24, p1);
    const f32x2_t sv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s, 1.0f, false);
    acc = __builtin_fmaf(p0, sv[0], acc);
    return __builtin_fmaf(p1, sv[1], acc);
  } else if constexpr (Traits<F>::kBits == 4) {
    float p = dot8_f32<F>(c.x, 0u, xf + 0, 0.0f);
    p = dot8_f32<F>(c.y, 0u, xf + 8, p);
    p = dot8_f32<F>(c.z, 0u, xf + 16, p);
    p = dot8_f32<F>(c.w, 0u, xf + 24, p);
    acc = __builtin_fmaf(p, block_scale<F>(s), acc);
    if constexpr (F == kINT4_AFFINE) {
      float xs = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) xs += xf[i];
      acc = __builtin_fmaf(xs, bf16_bits_to_f32(b), acc);
    }
    return acc;
  } else {
    float p = dot8_f32<F>(c.x, c.y, xf + 0, 0.0f);
    p = dot8_f32<F>(c.z, c.w, xf + 8, p);
    return __builtin_fmaf(p, block_scale<F>(s), acc);
  }
}

// Launch parameters, with the per-row byte counts and the chunk count worked
// out on the host (the kernel does no division by a runtime value).
struct GemvParams {
  const uint8_t *codes;
  const uint8_t *scales;
  const uint16_t *biases;
  const uint16_t *x;
  void *out;
  const int32_t *eids;
  int *status;
  int64_t n, k, nexp;  // output rows, reduction length, experts in the stack
  uint64_t rowb;       // code bytes per weight row
  uint64_t srowb;      // scale bytes per weight row
  float global;
  int ot;              // 0: f32 out, 1: bf16 out
  int C;               // 16-byte code chunks per row
  const uint16_t *g;   // fused RMSNorm: the norm weight (bf16 [k]), and its eps
  float eps;
};

// O32: every code and scale byte offset of the (stacked) weight fits in 31
// bits, so all index arithmetic is unsigned 32-bit and rows are addressed as
// a 32-bit offset from the weight's base (global_load with a scalar base and
// a vector offset).  The per-wave set-up before the first load is what every
// wave of a CU waits behind on the shared scalar unit: with 64-bit row
// pointers and signed 64-bit divisions it was ~160 scalar instructions per
// wave (nvfp4 4096 x 4096: 4.06 us).
// ONE: every wave has exactly one full round (k = 64 * KW chunks), so the
// round loop, its guards and their scalar set-up drop out.
template <int F, int KW, int R, int S, int WPG, bool O32, bool ONE>
__global__ void __launch_bounds__(WPG * 64) gemv_kernel(const GemvParams p) {
  constexpr int E = kE<F>, XQ = E / 8, RG = WPG / KW, RS = R * S;
  constexpr int SB = (F == kNVFP8 || F == kINT8_SYM) ? 4 : (F == kINT4_AFFINE ? 2 : 1);  // bytes per scale
  typedef typename std::conditional<O32, uint32_t, uint64_t>::type idx_t;
  static_assert(WPG % KW == 0 && (KW & (KW - 1)) == 0, "k split: a power of two dividing the waves");
  const int lane = threadIdx.x & 63;
  const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index: uniform
  const uint32_t rg = w / KW, ks = w % KW;
  // Set-up kept short and in 32-bit unsigned arithmetic on the O32 path: it
  // runs on the CU's shared scalar unit for every wave before its first load.
  const idx_t n = (idx_t)p.n;
  const idx_t rowb = (idx_t)p.rowb, srowb = (idx_t)p.srowb;
  const uint32_t C = (uint32_t)p.C;
  const uint32_t i = blockIdx.y;  // activation row
  const idx_t jb = ((idx_t)blockIdx.x * RG + rg) * RS;
  idx_t jbase = 0;
  bool skip = false;
  if (p.eids) {
    const int64_t e = p.eids[i];
    skip = e < 0 || e >= p.nexp;
    if (skip && p.status && blockIdx.x == 0 && threadIdx.x == 0) *p.status = 1;
    jbase = skip ? 0 : (idx_t)e * n;
  }
  const uint16_t *xr = p.x + (idx_t)i * (idx_t)p.k;
  __shared__ float red[KW > 1 ? WPG : 1][RS];

  float acc[S][R];
  idx_t coff[S][R], soff[S][R];  // byte offsets of each row's codes and scales
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc[s][r] = 0.0f;
      // rows past n read row n-1 and are never stored
      const idx_t jr = jbase + __builtin_elementwise_min(jb + (idx_t)(s * R + r), n - 1);
      coff[s][r] = jr * rowb;
      soff[s][r] = jr * srowb;
    }

  // One round: lane l of this wave takes chunk base + l of every row of the
  // group.  Full rounds carry no bounds checks; the last (guarded) round of a
  // wave masks chunks past the row.
  auto store = [&](idx_t j, float v) {
    if constexpr (F == kNVFP4) v *= p.global;
    const uint64_t o = (uint64_t)i * (uint64_t)n + j;
    if (p.ot == 0) reinterpret_cast<float *>(p.out)[o] = v;
    else reinterpret_cast<uint16_t *>(p.out)[o] = f32_to_bf16_bits(v);
  };
  // Group s is complete: reduce its R rows jointly and store them (KW == 1)
  // or leave them in LDS for the k-split combine.
  auto finish = [&](int s) {
    const float v = joint_sum<R>(acc[s]);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (lane == out_lane<R>(r)) {
        if constexpr (KW == 1) {
          if (jb + s * R + r < n) store(jb + s * R + r, v);
        } else {
          red[w][s * R + r] = v;
        }
      }
    }
  };

  auto round = [&](auto guard, auto last, uint32_t base) {
    constexpr bool kG = decltype(guard)::value;
    constexpr bool kLast = decltype(last)::value;
    const uint32_t ch = base + lane;
    const bool in = !kG || ch < C;
    const uint32_t cc = in ? ch : 0u;
    uint4 xq[XQ];
    v4u cw[S][R];
    uint32_t sw[S][R], bw[S][R];
    auto load_group = [&](int s) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        cw[s][r] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p.codes + (coff[s][r] + (idx_t)cc * 16)));
#pragma unroll
      for (int r = 0; r < R; ++r) {
        bw[s][r] = 0u;
        load_sc<F>(p.scales + soff[s][r], p.biases + soff[s][r] / SB, cc, sw[s][r], bw[s][r]);
      }
    };
    // Issue order (fenced): the first group's codes and scales, then x, then
    // the later groups.  The HBM requests leave first; x (an L2 hit) must not
    // hold them back in the address unit, and it still arrives before the
    // first group is consumed, so the in-order wait for that group covers it.
    load_group(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < XQ; ++q) xq[q] = reinterpret_cast<const uint4 *>(xr + (idx_t)cc * E)[q];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 1; s < S; ++s) load_group(s);
    // every load of the round is in flight before the first use
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (in) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          // An empty asm that reads and writes the loaded words pins their
          // first use here: otherwise instruction selection may place the
          // scale decode right after its load, and the wait it needs would
          // hold back the loads issued after it.
          asm volatile("" : "+v"(cw[s][r]), "+v"(sw[s][r]));
          acc[s][r] = chunk_dot<F>(cw[s][r], sw[s][r], bw[s][r], xq, acc[s][r]);
        }
      }
      // in the wave's last round a group's sums are final as soon as its dots
      // are: its reduction overlaps the arrival of the later groups' data
      if constexpr (kLast) finish(s);
    }
  };
  // rounds whose 64 chunks all lie inside the row, then at most one partial;
  // the wave's last round finishes each group as it goes
  constexpr uint32_t step = 64 * KW;
  const uint32_t first = ks * 64;
  constexpr std::integral_constant<bool, false> kNo{};
  constexpr std::integral_constant<bool, true> kYes{};
  if constexpr (ONE) {
    if (!skip) {
      round(kNo, kYes, first);
    } else {
#pragma unroll
      for (int s = 0; s < S; ++s) finish(s);
    }
  } else {
  const uint32_t nfull = skip ? 0u : (C >= first + 64 ? (C - first - 64) / step + 1 : 0u);
  const bool partial = !skip && first + nfull * step < C;
  if (partial) {
    for (uint32_t rr = 0; rr < nfull; ++rr) round(kNo, kNo, first + rr * step);
    round(kYes, kYes, first + nfull * step);
  } else if (nfull > 0) {
    for (uint32_t rr = 0; rr + 1 < nfull; ++rr) round(kNo, kNo, first + rr * step);
    round(kNo, kYes, first + (nfull - 1) * step);
  } else {
    // no chunk for this wave (a bad expert id, or k shorter than the split)
#pragma unroll
    for (int s = 0; s < S; ++s) finish(s);
  }
  }
  if constexpr (KW > 1) {
    __syncthreads();
    if (ks == 0 && lane < RS && jb + lane < n) {
      float t = 0.0f;
#pragma unroll
      for (int q = 0; q < KW; ++q) t += red[rg * KW + q][lane];
      store(jb + lane, t);
    }
  }
}

// One-round kernel: every wave covers its k split in a single round (the row
// is exactly 64 * KW chunks: k = 4096 for both code widths).  Written with
// plain per-lane 32-bit index arithmetic and 64-bit lane pointers; measured
// faster than the general kernel with its single round selected at compile
// time (nvfp4 4096 x 4096: 3.65 vs 3.9 us; the set-up of the general kernel,
// scalar row offsets and scalar-base loads, costs the difference).
// NORM: the fused RMSNorm (one bf16 row): each lane also loads its chunk of
// the norm weight g, multiplies x * g in f32 (exact for bf16 inputs) and sums
// x^2; the dots run against x * g in f32, and the row's 1 / sqrt(mean x^2 +
// eps) scales each output once, after the sums of x^2 of the k-split waves
// meet in LDS with the dots.
template <int F, int KW, int R, int S, int WPG, bool NORM = false>
__global__ void __launch_bounds__(WPG * 64) gemv1_kernel(const GemvParams p) {
  constexpr int E = kE<F>, XQ = E / 8, RG = WPG / KW, RS = R * S;
  constexpr int SB = (F == kNVFP8 || F == kINT8_SYM) ? 4 : (F == kINT4_AFFINE ? 2 : 1);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rg = w / KW, ks = w - rg * KW;
  const int n = (int)p.n;
  const int rowb = (int)p.rowb, srowb = (int)p.srowb;
  const int i = blockIdx.y;
  const int j0 = (blockIdx.x * RG + rg) * RS;
  const int ch = ks * 64 + lane;
  int jbase = 0;
  bool skip = false;
  if (p.eids) {
    const int e = p.eids[i];
    skip = e < 0 || (int64_t)e >= p.nexp;
    if (skip && p.status && blockIdx.x == 0 && threadIdx.x == 0) *p.status = 1;
    jbase = skip ? 0 : e * n;
  }
  __shared__ float red[KW > 1 ? WPG : 1][RS + (NORM ? 1 : 0)];
  v4u cw[S][R];
  uint32_t sw[S][R], bw[S][R];
  uint4 xq[XQ];
  uint4 gq[NORM ? XQ : 1];
  float acc[S][R];
  auto load_group = [&](int s) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int jr = jbase + min(j0 + s * R + r, n - 1);  // rows past n: read row n-1, never stored
      bw[s][r] = 0u;
      load_sc<F>(p.scales + (size_t)jr * srowb, p.biases + (size_t)jr * (srowb / SB), (uint32_t)ch, sw[s][r], bw[s][r]);
      cw[s][r] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p.codes + (size_t)jr * rowb) + ch);
    }
  };
  if (!skip) {
    load_group(0);
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t *xr = p.x + (size_t)i * (size_t)p.k;
#pragma unroll
    for (int q = 0; q < XQ; ++q) xq[q] = reinterpret_cast<const uint4 *>(xr + ch * E)[q];
    if constexpr (NORM) {
#pragma unroll
      for (int q = 0; q < XQ; ++q) gq[q] = reinterpret_cast<const uint4 *>(p.g + ch * E)[q];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 1; s < S; ++s) load_group(s);
    __builtin_amdgcn_sched_barrier(0);
  }
  // NORM: x * g and this lane's share of sum x^2
  float xg[NORM ? E : 1];
  float ssq = 0.0f;
  if constexpr (NORM) {
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      const uint32_t xv[4] = {xq[q].x, xq[q].y, xq[q].z, xq[q].w}, gv[4] = {gq[q].x, gq[q].y, gq[q].z, gq[q].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float x0 = __uint_as_float(xv[t] << 16), x1 = __uint_as_float(xv[t] & 0xFFFF0000u);
        xg[8 * q + 2 * t] = x0 * __uint_as_float(gv[t] << 16);
        xg[8 * q + 2 * t + 1] = x1 * __uint_as_float(gv[t] & 0xFFFF0000u);
        ssq = __builtin_fmaf(x0, x0, ssq);
        ssq = __builtin_fmaf(x1, x1, ssq);
      }
    }
  }
  auto store = [&](int j, float v) {
    if constexpr (F == kNVFP4) v *= p.global;
    const size_t o = (size_t)i * (size_t)n + j;
    if (p.ot == 0) reinterpret_cast<float *>(p.out)[o] = v;
    else reinterpret_cast<uint16_t *>(p.out)[o] = f32_to_bf16_bits(v);
  };
#pragma unroll
  for (int s = 0; s < S; ++s) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc[s][r] = 0.0f;
      if (!skip) {
        asm volatile("" : "+v"(cw[s][r]), "+v"(sw[s][r]));
        if constexpr (NORM) acc[s][r] = chunk_dot_f32<F>(cw[s][r], sw[s][r], bw[s][r], xg, 0.0f);
        else acc[s][r] = chunk_dot<F>(cw[s][r], sw[s][r], bw[s][r], xq, 0.0f);
      }
    }
    const float v = joint_sum<R>(acc[s]);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (lane == out_lane<R>(r)) {
        if constexpr (KW == 1) {
          if (j0 + s * R + r < n) store(j0 + s * R + r, v);
        } else {
          red[w][s * R + r] = v;
        }
      }
    }
  }
  static_assert(!NORM || KW > 1, "the fused norm's sums meet in the k-split reduction");
  if constexpr (NORM) {
    const float tq = wave_sum(ssq);
    if (lane == 0) red[w][RS] = tq;
  }
  if constexpr (KW > 1) {
    __syncthreads();
    if (ks == 0 && lane < RS && j0 + lane < n) {
      float t = 0.0f;
#pragma unroll
      for (int q = 0; q < KW; ++q) t += red[rg * KW + q][lane];
      if constexpr (NORM) {
        float sq = 0.0f;
#pragma unroll
        for (int q = 0; q < KW; ++q) sq += red[rg * KW + q][RS];
        t *= 1.0f / sqrtf(sq / (float)p.k + p.eps);
      }
      store(j0 + lane, t);
    }
  }
}

// The decode form of the expert-grouped matmul: one pass over an expert's
// weight rows serves up to T of the rows routed to it, where the per-row
// gather streams the expert once per routed row.
//
// The routing is done in the kernel (m <= 32): each wave reads the ids
// through the scalar unit, lane j counts the earlier rows with row j's
// expert, and the valid rows whose count is a multiple of T become tile
// leaders (one ballot); a tile is its leader and the next T - 1 rows (in row
// order) of the leader's expert, found from ballots, so the tile is uniform.
// Grid y enumerates the leaders; workgroups past their number exit after the
// id loads.  Rows whose id is outside [0, E) are zeroed by the workgroups of
// y = 0, which set *status to 1.
//
// Each tile runs the body for its own row count (1, 2 or 4 rows; 3 takes the
// 4-row body with its last row repeated and not stored), so a lone row does
// one row's loads and arithmetic.  Same geometry as the per-row kernels: one
// round when k is 64 chunks per wave of the k split (k = 4096), else
// guarded rounds as in gemv_kernel.  Every lane holds its chunk's activations
// of the tile's rows, and the weight chunk is decoded once for all of them
// (the conversions are pure operations on the same words, so the compiler
// emits them once).
template <int F, int KW, int R, int S, int WPG, int T, bool ONE>
__device__ __forceinline__ void gemvg_body(const GemvParams &p, const int (&tok)[4], int nr, int e,
                                           float (*red)[R * S * 4]) {
  constexpr int E = kE<F>, XQ = E / 8, RG = WPG / KW, RS = R * S;
  constexpr int SB = (F == kNVFP8 || F == kINT8_SYM) ? 4 : (F == kINT4_AFFINE ? 2 : 1);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rg = w / KW, ks = w - rg * KW;
  const int n = (int)p.n;
  const int rowb = (int)p.rowb, srowb = (int)p.srowb;
  const int j0 = (blockIdx.x * RG + rg) * RS;
  const int jbase = e * n;
  float acc[S][T][R];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[s][t][r] = 0.0f;
  // Group s is complete: reduce its R rows jointly for every tile row and
  // leave the sums in LDS for the k-split combine.
  auto finish = [&](int s) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float v = joint_sum<R>(acc[s][t]);
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (lane == out_lane<R>(r)) red[w][t * RS + s * R + r] = v;
    }
  };
  // One round: lane l takes chunk ch of every row of the wave's groups (a
  // chunk past the row, in a wave's last round, loads chunk 0 and adds
  // nothing).  In the wave's last round each group is reduced as soon as its
  // dots are done, overlapping the arrival of the later groups' data.
  auto round = [&](int ch, bool in, bool last) {
    const int cc = in ? ch : 0;
    v4u cw[S][R];
    uint32_t sw[S][R], bw[S][R];
    uint4 xq[T][XQ];
    auto load_group = [&](int s) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int jr = jbase + min(j0 + s * R + r, n - 1);  // rows past n: read row n-1, never stored
        bw[s][r] = 0u;
        load_sc<F>(p.scales + (size_t)jr * srowb, p.biases + (size_t)jr * (srowb / SB), (uint32_t)cc, sw[s][r],
                   bw[s][r]);
        cw[s][r] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p.codes + (size_t)jr * rowb) + cc);
      }
    };
    load_group(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const uint16_t *xr = p.x + (size_t)tok[t] * (size_t)p.k;
#pragma unroll
      for (int q = 0; q < XQ; ++q) xq[t][q] = reinterpret_cast<const uint4 *>(xr + cc * E)[q];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 1; s < S; ++s) load_group(s);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (ONE || in) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          asm volatile("" : "+v"(cw[s][r]), "+v"(sw[s][r]));
#pragma unroll
          for (int t = 0; t < T; ++t) acc[s][t][r] = chunk_dot<F>(cw[s][r], sw[s][r], bw[s][r], xq[t], acc[s][t][r]);
        }
      }
      if (ONE || last) finish(s);
    }
  };
  if constexpr (ONE) {
    round(ks * 64 + lane, true, true);
  } else {
    // this wave's rounds: chunks ks * 64 + lane + i * 64 * KW below C
    const int C = p.C, first = ks * 64;
    const int nround = C > first ? (C - first + 64 * KW - 1) / (64 * KW) : 0;
    for (int i = 0; i + 1 < nround; ++i) round(first + i * 64 * KW + lane, true, false);
    if (nround > 0) {
      const int ch = first + (nround - 1) * 64 * KW + lane;
      round(ch, ch < C, true);
    } else {
#pragma unroll
      for (int q = 0; q < S; ++q) finish(q);  // k shorter than the split: this wave adds zeros
    }
  }
  __syncthreads();
  if (ks == 0 && lane < RS * T) {
    const int t = lane / RS, jj = lane - t * RS;
    if (t < nr && j0 + jj < n) {
      float v = 0.0f;
#pragma unroll
      for (int q = 0; q < KW; ++q) v += red[rg * KW + q][lane];
      if constexpr (F == kNVFP4) v *= p.global;
      const size_t o = (size_t)tok[t] * (size_t)n + j0 + jj;
      if (p.ot == 0) reinterpret_cast<float *>(p.out)[o] = v;
      else reinterpret_cast<uint16_t *>(p.out)[o] = f32_to_bf16_bits(v);
    }
  }
}

template <int F, int KW, int R, int S, int WPG, bool ONE>
__global__ void __launch_bounds__(WPG * 64) gemvg_kernel(const GemvParams p, int m) {
  constexpr int T = kGemvGroupRows, RG = WPG / KW, RS = R * S;
  static_assert(KW > 1 && T == 4 && RS * T <= 64, "the k-split combine stores one sum per lane");
  __shared__ float red[WPG][RS * T];
  int tok[4], nr, e;
  if (!p.eids) {
    // dense rows of one weight (no routing): tile y is rows 4y .. 4y + 3 below m
    const int r0 = blockIdx.y * T;
    nr = min(T, m - r0);
#pragma unroll
    for (int t = 0; t < 4; ++t) tok[t] = r0 + min(t, nr - 1);
    e = 0;
  } else {
    constexpr int MM = (int)kGemvGroupMaxRows;
    const int lane = threadIdx.x & 63;
    // The ids through the scalar unit: uniform loads that, after the first
    // workgroup on a CU, hit its scalar cache, so a workgroup with no tile
    // leaves after a short wait.  Lane j takes row j's expert and counts the
    // earlier rows of the same expert.
    int ids[MM];
#pragma unroll
    for (int j = 0; j < MM; ++j) ids[j] = j < m ? p.eids[j] : -1;
    int el = -1, rank = 0;
#pragma unroll
    for (int j = 0; j < MM; ++j) el = lane == j ? ids[j] : el;
#pragma unroll
    for (int j = 0; j < MM; ++j) rank += (j < lane && ids[j] == el) ? 1 : 0;
    const bool valid = lane < m && el >= 0 && (int64_t)el < p.nexp;
    if (blockIdx.y == 0) {
      const uint64_t bad = __ballot(lane < m && !valid);
      if (bad) {
        if (p.status && blockIdx.x == 0 && threadIdx.x == 0) *p.status = 1;
        const int c0 = blockIdx.x * RG * RS, n = (int)p.n;
        for (uint64_t b = bad; b; b &= b - 1) {
          const int i = __builtin_ctzll(b);
          for (int c = threadIdx.x; c < RG * RS && c0 + c < n; c += WPG * 64) {
            const size_t o = (size_t)i * (size_t)n + c0 + c;
            if (p.ot == 0) reinterpret_cast<float *>(p.out)[o] = 0.0f;
            else reinterpret_cast<uint16_t *>(p.out)[o] = 0;
          }
        }
      }
    }
    uint64_t lead = __ballot(valid && rank % T == 0);
    if ((int)blockIdx.y >= __popcll(lead)) return;  // uniform: no tile for this y
    for (unsigned q = 0; q < blockIdx.y; ++q) lead &= lead - 1;
    const int p0 = __builtin_ctzll(lead);
    e = __builtin_amdgcn_readlane(el, p0);
    uint64_t same = (__ballot(valid && el == e) >> p0) & ~(uint64_t)1;  // the expert's rows after the leader
    tok[0] = tok[1] = tok[2] = tok[3] = p0;
    nr = 1;
#pragma unroll
    for (int t = 1; t < 4; ++t) {
      tok[t] = same ? p0 + __builtin_ctzll(same) : tok[t - 1];
      nr += same ? 1 : 0;
      same &= same - 1;
    }
  }
  if (nr == 1) gemvg_body<F, KW, R, S, WPG, 1, ONE>(p, tok, nr, e, red);
  else if (nr == 2) gemvg_body<F, KW, R, S, WPG, 2, ONE>(p, tok, nr, e, red);
  else gemvg_body<F, KW, R, S, WPG, 4, ONE>(p, tok, nr, e, red);
}

// Measured on MI355X (graph replay, cold weights, nvfp4 4096 x 4096, us per
// launch on one box): 4-bit codes take KW = 2 and four sequential groups of 2
// rows per wave pair in 4-wave workgroups, 16 rows each (3.75; the same 16
// rows as two groups in 8-wave workgroups 3.88, one group of 2 rows 4.12,
// 3 / 6 / 8 groups 4.26 / 4.25 / 4.73, groups of 4 rows 4.08-4.75, 2- or
// 16-wave workgroups 4.26-4.7; the one-wave-per-row-pair kernel 4.76); the
// fused RMSNorm and the routed gather gain with it (4.99 -> 4.48, 23.6 ->
// 22.7).  8-bit codes take KW = 4, one group of 2 rows, 4 waves (mxfp8 14336
// x 4096: 10.4 us against a 10.1 us pure read of the codes).
template <int F>
GemvParams params(const QWeight &w, const void *x, void *out, int ot) {
  constexpr bool k4 = Traits<F>::kBits == 4;
  constexpr int SB = (F == kNVFP8 || F == kINT8_SYM) ? 4 : (F == kINT4_AFFINE ? 2 : 1);
  GemvParams p{};
  p.codes = (const uint8_t *)w.codes;
  p.scales = (const uint8_t *)w.scales;
  p.biases = (const uint16_t *)w.biases;
  p.x = (const uint16_t *)x;
  p.out = out;
  p.n = w.n;
  p.k = w.k;
  p.rowb = (uint64_t)(k4 ? w.k / 2 : w.k);
  p.srowb = (uint64_t)(w.k / Traits<F>::kBlock) * SB;
  p.global = w.global;
  p.ot = ot;
  p.C = (int)(w.k / (k4 ? 32 : 16));
  return p;
}

template <int F>
hipError_t run(const QWeight &w, int64_t m, const void *x, void *out, int ot, const int32_t *eids, int64_t nexp,
               int *status, hipStream_t s, const void *gam = nullptr, float eps = 0.0f) {
  constexpr bool k4 = Traits<F>::kBits == 4;
  constexpr int KW = k4 ? 2 : 4, R = 2, S = k4 ? 4 : 1, WPG = 4;
  constexpr int rows_per_wg = (WPG / KW) * R * S;
  const int64_t wgs = (w.n + rows_per_wg - 1) / rows_per_wg;
  if (wgs > 0x7FFFFFFF || m > 65535) return hipErrorInvalidValue;
  GemvParams p = params<F>(w, x, out, ot);
  p.eids = eids;
  p.status = status;
  p.nexp = nexp;
  p.g = (const uint16_t *)gam;
  p.eps = eps;
  const int64_t total_rows = w.n * (eids ? nexp : 1);
  // 32-bit offsets: the codes (scales are smaller) and the activation rows
  const bool o32 = total_rows * (int64_t)p.rowb < ((int64_t)1 << 31) && m * w.k < ((int64_t)1 << 30);
  const bool one = p.C == 64 * KW;
  const dim3 grid((unsigned)wgs, (unsigned)m), block(WPG * 64);
  if (gam) {  // the fused RMSNorm: the one-round kernel only (checked by gemv_norm_applies)
    if (!(o32 && one)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemv1_kernel<F, KW, R, S, WPG, true>), grid, block, 0, s, p);
    return hipGetLastError();
  }
  if (o32 && one) hipLaunchKernelGGL((gemv1_kernel<F, KW, R, S, WPG>), grid, block, 0, s, p);
  else if (o32) hipLaunchKernelGGL((gemv_kernel<F, KW, R, S, WPG, true, false>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((gemv_kernel<F, KW, R, S, WPG, false, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

// The grouped decode form: the geometry of run(), one grid row per possible
// tile.
template <int F>
hipError_t run_grouped(const QWeight &w, int64_t m, int64_t nexp, const int32_t *eids, const void *x, void *out,
                       int ot, int *status, hipStream_t s) {
  constexpr bool k4 = Traits<F>::kBits == 4;
  constexpr int KW = k4 ? 2 : 4, R = 2, S = k4 ? 4 : 1, WPG = 4;
  constexpr int rows_per_wg = (WPG / KW) * R * S;
  const int64_t wgs = (w.n + rows_per_wg - 1) / rows_per_wg;
  if (wgs > 0x7FFFFFFF || m < 1 || m > kGemvGroupMaxRows) return hipErrorInvalidValue;
  GemvParams p = params<F>(w, x, out, ot);
  p.eids = eids;
  p.nexp = nexp;
  p.status = status;
  // routed tiles: sum over the D routed experts of ceil(rows / T) <= (m + (T - 1) D) / T, D <= min(E, m);
  // and <= m.  Dense rows (no ids): ceil(m / T) tiles.
  constexpr int T = kGemvGroupRows;
  const int64_t tiles = eids ? std::min<int64_t>(m, (m + (T - 1) * std::min(nexp, m)) / T) : (m + T - 1) / T;
  if (p.C == 64 * KW)
    hipLaunchKernelGGL((gemvg_kernel<F, KW, R, S, WPG, true>), dim3((unsigned)wgs, (unsigned)tiles), dim3(WPG * 64),
                       0, s, p, (int)m);
  else
    hipLaunchKernelGGL((gemvg_kernel<F, KW, R, S, WPG, false>), dim3((unsigned)wgs, (unsigned)tiles), dim3(WPG * 64),
                       0, s, p, (int)m);
  return hipGetLastError();
}

}  // namespace

bool gemv_grouped_applies(const QWeight &w, int64_t m, int64_t nexp) {
  // decode-sized m, whole 16-byte code chunks, 31-bit offsets of the stacked weight and of x
  const int64_t E = is_4bit(w.fmt) ? 32 : 16, rowb = is_4bit(w.fmt) ? w.k / 2 : w.k;
  return m >= 1 && m <= kGemvGroupMaxRows && w.k >= E && w.k % E == 0 && w.n * nexp * rowb < ((int64_t)1 << 31) &&
         m * w.k < ((int64_t)1 << 30);
}

bool gemv_dense_preferred(const QWeight &w, int64_t m) {
  if (m > kGemvDenseRows || !gemv_grouped_applies(w, m, 1)) return false;
  if (m <= 8) return true;
  // packed bytes of the weight: codes, scales (and int4 biases)
  const int64_t B = block_of(w.fmt), sb = (w.fmt == kNVFP8 || w.fmt == kINT8_SYM) ? 4 : (w.fmt == kINT4_AFFINE ? 2 : 1);
  const int64_t row = (is_4bit(w.fmt) ? w.k / 2 : w.k) + (w.k / B) * sb + (w.fmt == kINT4_AFFINE ? (w.k / B) * 2 : 0);
  return (m + kGemvGroupRows - 1) / kGemvGroupRows * w.n * row <= (int64_t)96 << 20;
}

hipError_t launch_gemv_grouped(const QWeight &w, int64_t m, int64_t nexp, const int32_t *eids, const void *x,
                               void *out, int ot, int *status, hipStream_t s) {
  switch (w.fmt) {
    case kMXFP4: return run_grouped<kMXFP4>(w, m, nexp, eids, x, out, ot, status, s);
    case kNVFP4: return run_grouped<kNVFP4>(w, m, nexp, eids, x, out, ot, status, s);
    case kMXFP8_E4M3: return run_grouped<kMXFP8_E4M3>(w, m, nexp, eids, x, out, ot, status, s);
    case kMXFP8_E5M2: return run_grouped<kMXFP8_E5M2>(w, m, nexp, eids, x, out, ot, status, s);
    case kNVFP8: return run_grouped<kNVFP8>(w, m, nexp, eids, x, out, ot, status, s);
    case kINT4_AFFINE: return run_grouped<kINT4_AFFINE>(w, m, nexp, eids, x, out, ot, status, s);
    case kINT8_SYM: return run_grouped<kINT8_SYM>(w, m, nexp, eids, x, out, ot, status, s);
  }
  return hipErrorInvalidValue;
}

bool gemv_applies(const QWeight &w, int64_t m, int xt, bool routed) {
  // bf16 activations, whole 16-byte code chunks, one weight pass per row
  const int64_t E = is_4bit(w.fmt) ? 32 : 16;
  return xt == 1 && w.k % E == 0 && w.k / E < ((int64_t)1 << 30) && (m == 1 || routed);
}

bool gemv_norm_applies(const QWeight &w, int64_t m, int xt) {
  // up to kGemvNormRows bf16 rows (one grid row each; their weight passes meet in the caches),
  // one full round of 16-byte chunks per wave (k = 4096), 31-bit offsets
  const bool k4 = is_4bit(w.fmt);
  const int64_t E = k4 ? 32 : 16, KW = k4 ? 2 : 4;
  return xt == 1 && m >= 1 && m <= kGemvNormRows && w.k == 64 * KW * E &&
         w.n * (k4 ? w.k / 2 : w.k) < ((int64_t)1 << 31);
}

hipError_t launch_gemv_norm(const QWeight &w, int64_t m, const void *x, const void *gam, float eps, void *out, int ot,
                            hipStream_t s) {
  switch (w.fmt) {
    case kMXFP4: return run<kMXFP4>(w, m, x, out, ot, nullptr, 0, nullptr, s, gam, eps);
    case kNVFP4: return run<kNVFP4>(w, m, x, out, ot, nullptr, 0, nullptr, s, gam, eps);
    case kMXFP8_E4M3: return run<kMXFP8_E4M3>(w, m, x, out, ot, nullptr, 0, nullptr, s, gam, eps);
    case kMXFP8_E5M2: return run<kMXFP8_E5M2>(w, m, x, out, ot, nullptr, 0, nullptr, s, gam, eps);
    case kNVFP8: return run<kNVFP8>(w, m, x, out, ot, nullptr, 0, nullptr, s, gam, eps);
    case kINT4_AFFINE: return run<kINT4_AFFINE>(w, m, x, out, ot, nullptr, 0, nullptr, s, gam, eps);
    case kINT8_SYM: return run<kINT8_SYM>(w, m, x, out, ot, nullptr, 0, nullptr, s, gam, eps);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(const QWeight &w, int64_t m, const void *x, void *out, int ot, const int32_t *eids,
                       int64_t nexp, int *status, hipStream_t s) {
  switch (w.fmt) {
    case kMXFP4: return run<kMXFP4>(w, m, x, out, ot, eids, nexp, status, s);
    case kNVFP4: return run<kNVFP4>(w, m, x, out, ot, eids, nexp, status, s);
    case kMXFP8_E4M3: return run<kMXFP8_E4M3>(w, m, x, out, ot, eids, nexp, status, s);
    case kMXFP8_E5M2: return run<kMXFP8_E5M2>(w, m, x, out, ot, eids, nexp, status, s);
    case kNVFP8: return run<kNVFP8>(w, m, x, out, ot, eids, nexp, status, s);
    case kINT4_AFFINE: return run<kINT4_AFFINE>(w, m, x, out, ot, eids, nexp, status, s);
    case kINT8_SYM: return run<kINT8_SYM>(w, m, x, out, ot, eids, nexp, status, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace bsq
