// mfma.hip -- prefill qgemm on gfx950 matrix cores (bf16 X):
//   out[i,j] = sum_p X[i,p] * dequant(W)[j,p].
//
// This is the dense contraction of the method [metaltile PR #250,
// "mt_mxfp4_qmm_mma" (the M >= 32 path) and the MMA commits for all formats;
// metaltile-std src/mlx/fp_quantized_mma.rs, mt_fp4_qmm_mma: stage X and
// dequantized W per k-block, then multiply-accumulate].  The Apple geometry
// (32x32x32 tiles, 8x8 simdgroup fragments) is not used; the CDNA4 design:
//
//  * v_mfma_f32_32x32x16_bf16, fp32 accumulators in registers.  Operand
//    layout for 32x32x16: lane l holds row/column l%32 and the 8 consecutive
//    k values 8*(l/32)..8*(l/32)+7 of the 16-deep slice; the accumulator lane
//    l holds column l%32, rows 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
//  * A workgroup owns a BM x BN output tile; its waves split it WGM x WGN.
//    The k loop steps BK = 64.  Inside a step the 16-deep MFMA slices are
//    k-permuted: slice t, lane half h covers k = 32h + 8t + (0..7).  Both
//    operands use the same permutation, so the sum is unchanged, and each
//    lane's weight codes for a step are one contiguous 16-byte (4-bit) or
//    32-byte (8-bit) run that maps straight onto its B-operand registers.
//  * X (bf16) goes global -> registers -> LDS (rows padded to 144 bytes so
//    the 16-byte fragment reads are bank-conflict free) and is read back as A
//    fragments.  Large problems use three X buffers and the step-ahead
//    schedule (SCHED 5): step kt+1 is already in LDS while step kt runs, so
//    its first fragments and its weight decode happen during step kt and the
//    MFMAs never wait on the barrier; 8 waves (two per SIMD) per 256x128 tile.
//  * W codes go global -> registers and are decoded there into bf16 B
//    fragments, never touching LDS:
//      mxfp4 / mxfp8:  v_cvt_scalef32_pk_bf16_{fp4,fp8,bf8} with the E8M0
//                      scale (an exponent-only operand), exact in bf16;
//      nvfp4:          e2m1 * e4m3 micro-scale in f32 (exact, <= 6 significant
//                      bits) then bf16; the f32 global scales the accumulator
//                      once at the end ("global scale multiplied once at the
//                      end" [rlx-cpu quant.rs, dequant_matmul_nvfp4]);
//      int8 / int4 (step-ahead schedule): the integer codes, exact in bf16,
//                      into a per-block partial sum that gets the block scale
//                      once (int8: slices kept inside one 32-block by a second
//                      k permutation); int4's bias term b * sum x on the MFMA
//                      with the bias broadcast as the B operand;
//      nvfp8 (and int8 / int4 in the small-tile schedule): the f32
//                      dequantized value w (one rounding, as the standalone
//                      dequant) split into bf16 hi + lo, two MFMAs per slice;
//                      |w - hi - lo| <= 2^-17 |w|.
//  * Workgroup -> tile mapping is XCD-aware: consecutive workgroups are
//    dispatched round-robin over the 8 XCDs, so tiles are renumbered to give
//    each XCD a contiguous run of tiles that share X rows (one L2 per XCD).
#include "bsq_internal.hpp"
#include "codec.hpp"
#include "epilogue.hpp"

#include <type_traits>

namespace bsq {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;

constexpr int BK = 64;
constexpr int LDS_LD = BK + 8;  // bf16 per LDS row: 128 data bytes + 16 pad

template <int F> constexpr bool kSplit = (F == kNVFP8 || F == kINT8_SYM || F == kINT4_AFFINE);
// int8 / int4 in the step-ahead kernel instead: the integer codes go to the
// MFMA as they are (bf16 holds every q exactly), a per-block partial sum P is
// formed in fp32 and the block's scale is applied to P once, not per element
// (as rlx-cpu quant.rs dequant_matmul_int8 applies each block scale a single time):
// int8 acc += s_blk * P_blk, one MFMA per slice instead of the hi + lo pair.
// int4 (value s*q + b, one 64-group per step): acc += s * P after the step,
// and the bias term b * sum x (the split s*sum q*x + b*sum x of metaltile-std
// tests/qmm_gpu_correctness.rs cpu_qmm_reference) straight on the MFMA with
// the group's bias, exact in bf16, broadcast as the B operand: still two
// MFMAs per slice, but no per-element dequantize and hi/lo split.
template <int F> constexpr bool kFold = (F == kINT8_SYM || F == kINT4_AFFINE);

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// hi = bf16(w), lo = bf16(w - hi) for two values; returns (hi pair, lo pair).
__device__ __forceinline__ void split_pk(float a, float b, uint32_t &hi, uint32_t &lo) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  const bf16x2_t h = {ha, hb};
  const bf16x2_t l = {(__bf16)(a - (float)ha), (__bf16)(b - (float)hb)};
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

__device__ __forceinline__ bf16x8_t frag(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint4 u = make_uint4(a, b, c, d);
  return __builtin_bit_cast(bf16x8_t, u);
}

// One lane's weight data for one BK step of one 32-column subtile.
struct WRaw {
  uint4 c0, c1;       // codes: c0 only for 4-bit; c0, c1 (32 bytes) for 8-bit
  uint32_t s0, s1;    // raw scale bits (u8 E8M0/E4M3, f32 bits, bf16 bits)
  uint32_t b0;        // int4 bias bits
};

template <int F, bool VEC, bool SC = true, bool P2 = false>
__device__ __forceinline__ void load_w(WRaw &r, const uint8_t *__restrict__ codes, const void *__restrict__ scales,
                                       const uint16_t *__restrict__ biases, int64_t col, int64_t k, int64_t kbase,
                                       bool tail) {
  constexpr int B = Traits<F>::kBlock;
  const int64_t nblk = k / B;
  // kbase = k0 + 32h: this lane's 32 contiguous k values.
  if constexpr (Traits<F>::kBits == 4) {
    const uint8_t *p = codes + col * (k / 2) + kbase / 2;
    if (VEC && !tail) {
      r.c0 = *reinterpret_cast<const uint4 *>(p);
    } else {
      uint32_t t[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) t[q] = (kbase + 8 * q < k) ? reinterpret_cast<const uint32_t *>(p)[q] : 0u;
      r.c0 = make_uint4(t[0], t[1], t[2], t[3]);
    }
    r.c1 = make_uint4(0, 0, 0, 0);
  } else {
    // P2: the lane's two 16-byte runs are 32 bytes apart (k0+16h and k0+32+16h)
    constexpr int O1 = P2 ? 32 : 16;
    const uint8_t *p = codes + col * k + kbase;
    if (!tail) {
      r.c0 = *reinterpret_cast<const uint4 *>(p);
      r.c1 = *reinterpret_cast<const uint4 *>(p + O1);
    } else {
      uint32_t t[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int off = q < 4 ? 4 * q : O1 + 4 * (q - 4);
        t[q] = (kbase + off < k) ? *reinterpret_cast<const uint32_t *>(p + off) : 0u;
      }
      r.c0 = make_uint4(t[0], t[1], t[2], t[3]);
      r.c1 = make_uint4(t[4], t[5], t[6], t[7]);
    }
  }
  if constexpr (!SC) return;
  int64_t b0 = kbase / B, b1 = (kbase + (P2 ? 32 : 16)) / B;
  if (tail) {
    b0 = b0 < nblk ? b0 : nblk - 1;
    b1 = b1 < nblk ? b1 : nblk - 1;
  }
  const int64_t s = col * nblk;
  if constexpr (F == kMXFP4 || F == kNVFP4 || F == kMXFP8_E4M3 || F == kMXFP8_E5M2) {
    const uint8_t *sp = reinterpret_cast<const uint8_t *>(scales) + s;
    r.s0 = sp[b0];
    r.s1 = (B == 16) ? sp[b1] : r.s0;
  } else if constexpr (F == kNVFP8 || F == kINT8_SYM) {
    const uint32_t *sp = reinterpret_cast<const uint32_t *>(scales) + s;
    r.s0 = sp[b0];
    r.s1 = (B == 16 || P2) ? sp[b1] : r.s0;
  } else {
    r.s0 = reinterpret_cast<const uint16_t *>(scales)[s + b0];
    r.s1 = r.s0;
    r.b0 = biases[s + b0];
  }
}

// Trip scales: one lane's scale (and bias) words for the four 64-k steps of
// one 256-k trip of its column, loaded with one or two wide loads instead of
// one small load per step.  Needs k % 256 == 0 (every trip whole and its words
// aligned).  nvfp8 (64 bytes of f32 scales per trip) keeps per-step loads.
template <int F> constexpr bool kTripSc = F != kNVFP8 && F != kINT8_SYM;
template <int F> constexpr int kTripWords =
    (F == kMXFP4 || F == kMXFP8_E4M3 || F == kMXFP8_E5M2) ? 2 : (F == kNVFP4 || F == kINT4_AFFINE) ? 4 : 8;

template <int F>
__device__ __forceinline__ void load_trip_sc(uint32_t (&v)[kTripWords<F>], const void *__restrict__ scales,
                                             const uint16_t *__restrict__ biases, int64_t col, int64_t k, int trip) {
  constexpr int B = Traits<F>::kBlock, BPT = 256 / B;  // blocks per trip
  const int64_t blk = col * (k / B) + (int64_t)trip * BPT;
  if constexpr (F == kMXFP4 || F == kMXFP8_E4M3 || F == kMXFP8_E5M2) {
    const uint2 t = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint8_t *>(scales) + blk);
    v[0] = t.x, v[1] = t.y;
  } else if constexpr (F == kNVFP4) {
    const uint4 t = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(scales) + blk);
    v[0] = t.x, v[1] = t.y, v[2] = t.z, v[3] = t.w;
  } else if constexpr (F == kINT8_SYM) {
    const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint32_t *>(scales) + blk);
    const uint4 a = p[0], b = p[1];
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
  } else if constexpr (F == kINT4_AFFINE) {
    const uint2 a = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(scales) + blk);
    const uint2 b = *reinterpret_cast<const uint2 *>(biases + blk);
    v[0] = a.x, v[1] = a.y, v[2] = b.x, v[3] = b.y;
  }
}

// The raw scale fields of step S (0..3) of a trip for lane half h (the lane's
// k range in that step starts 32h into it).
template <int F, int S, bool FOLD = false>
__device__ __forceinline__ void trip_sc(WRaw &r, const uint32_t (&v)[kTripWords<F>], int h) {
  if constexpr (F == kMXFP4 || F == kMXFP8_E4M3 || F == kMXFP8_E5M2) {
    r.s0 = (v[S >> 1] >> (8 * (2 * (S & 1) + h))) & 0xFFu;  // block 2S + h
  } else if constexpr (F == kNVFP4) {
    r.s0 = (v[S] >> (16 * h)) & 0xFFu;  // blocks 4S + 2h and 4S + 2h + 1
    r.s1 = (v[S] >> (16 * h + 8)) & 0xFFu;
  } else if constexpr (F == kINT8_SYM && FOLD) {
    r.s0 = v[2 * S];  // both blocks of the step, for every lane
    r.s1 = v[2 * S + 1];
  } else if constexpr (F == kINT8_SYM) {
    r.s0 = h ? v[2 * S + 1] : v[2 * S];  // block 2S + h
  } else if constexpr (F == kINT4_AFFINE) {
    r.s0 = (v[S >> 1] >> (16 * (S & 1))) & 0xFFFFu;  // block S
    r.b0 = (v[2 + (S >> 1)] >> (16 * (S & 1))) & 0xFFFFu;
  }
}

// Build the B fragments (hi, and lo for split formats) of the 4 k-slices.
// FOLD: the integer codes as bf16 (exact) and the step's fold factors fs:
// int8 the scales of its two 32-blocks; int4 the group's scale, with lo[0] the
// group's bias broadcast to all 8 k of the fragment.
template <int F, bool FOLD = false>
__device__ __forceinline__ void decode_w(const WRaw &r, bf16x8_t hi[4], bf16x8_t lo[4], float fs[2] = nullptr) {
  const uint32_t cw[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
  if constexpr (FOLD && F == kINT8_SYM) {
    fs[0] = __uint_as_float(r.s0);
    fs[1] = __uint_as_float(r.s1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = (float)(int)(int8_t)(uint8_t)(cw[2 * t + (i >> 2)] >> (8 * (i & 3)));
      hi[t] = frag(pk_bf16(q[0], q[1]), pk_bf16(q[2], q[3]), pk_bf16(q[4], q[5]), pk_bf16(q[6], q[7]));
    }
  } else if constexpr (FOLD && F == kINT4_AFFINE) {
    fs[0] = bf16_bits_to_f32(r.s0);
    fs[1] = 0.0f;
    const uint32_t bb = (r.b0 & 0xFFFFu) * 0x10001u;  // the bias bf16 in both halves
    lo[0] = frag(bb, bb, bb, bb);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // even nibbles and odd nibbles as bytes, then bytes to f32 (v_cvt_f32_ubyte, exact) and bf16
      const uint32_t ev = cw[t] & 0x0F0F0F0Fu, od = (cw[t] >> 4) & 0x0F0F0F0Fu;
      hi[t] = frag(pk_bf16((float)((ev >> 0) & 0xFFu), (float)((od >> 0) & 0xFFu)),
                   pk_bf16((float)((ev >> 8) & 0xFFu), (float)((od >> 8) & 0xFFu)),
                   pk_bf16((float)((ev >> 16) & 0xFFu), (float)((od >> 16) & 0xFFu)),
                   pk_bf16((float)((ev >> 24) & 0xFFu), (float)((od >> 24) & 0xFFu)));
    }
  } else if constexpr (F == kMXFP4) {
    const float sc = __uint_as_float(r.s0 << 23);  // exponent-only scale operand
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t w = cw[t];
      hi[t] = frag(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3)));
    }
  } else if constexpr (F == kMXFP8_E4M3 || F == kMXFP8_E5M2) {
    const float sc = __uint_as_float(r.s0 << 23);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t w0 = cw[2 * t], w1 = cw[2 * t + 1];
      if constexpr (F == kMXFP8_E4M3) {
        hi[t] = frag(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true)));
      } else {
        hi[t] = frag(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, sc, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, sc, true)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, sc, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, sc, true)));
      }
    }
  } else if constexpr (F == kNVFP4) {
    const float m0 = e4m3_to_f32(r.s0), m1 = e4m3_to_f32(r.s1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float ms = t < 2 ? m0 : m1;  // slices 0,1 in the first 16-block
      const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[t], 1.0f, 0);
      const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[t], 1.0f, 1);
      const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[t], 1.0f, 2);
      const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[t], 1.0f, 3);
      // e2m1 * e4m3 has at most 6 significant bits: exact in f32 and in bf16
      hi[t] = frag(pk_bf16(v0[0] * ms, v0[1] * ms), pk_bf16(v1[0] * ms, v1[1] * ms), pk_bf16(v2[0] * ms, v2[1] * ms),
                   pk_bf16(v3[0] * ms, v3[1] * ms));
    }
  } else {
    // split formats: w = f32 dequantized value, then hi/lo bf16
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float w[8];
      if constexpr (F == kNVFP8) {
        const float s = __uint_as_float(t < 2 ? r.s0 : r.s1);
        const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw[2 * t], 1.0f, false);
        const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw[2 * t], 1.0f, true);
        const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw[2 * t + 1], 1.0f, false);
        const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw[2 * t + 1], 1.0f, true);
        const float e[8] = {v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = e[i] * s;
      } else if constexpr (F == kINT8_SYM) {
        const float s = __uint_as_float(r.s0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t word = cw[2 * t + (i >> 2)];
          const int q = (int)(int8_t)(uint8_t)(word >> (8 * (i & 3)));
          w[i] = (float)q * s;
        }
      } else {  // int4 affine: s*q + b
        const float s = bf16_bits_to_f32(r.s0), b = bf16_bits_to_f32(r.b0);
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = __builtin_fmaf(s, (float)((cw[t] >> (4 * i)) & 0xFu), b);
      }
      uint32_t h[4], l[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) split_pk(w[2 * i], w[2 * i + 1], h[i], l[i]);
      hi[t] = frag(h[0], h[1], h[2], h[3]);
      lo[t] = frag(l[0], l[1], l[2], l[3]);
    }
  }
}

// Calls fn(integral_constant<int, I>) for I = 0 .. N-1, in order.
template <int I, int N> struct Unroll {
  template <class Fn> __device__ __forceinline__ static void run(Fn &&fn) {
    if constexpr (I < N) {
      fn(std::integral_constant<int, I>{});
      Unroll<I + 1, N>::run(fn);
    }
  }
};

// Global data of one BK step held in registers: this thread's X chunks and
// this lane's weight words for each of its NT column subtiles.
template <int XCH, int NT>
struct Slot {
  uint4 x[XCH];
  WRaw w[NT];
};

// GRP (expert-grouped rows): gtab is the routing table the route kernel
// built: gtab[0] tiles in use, then per m-tile (expert, first row, row limit)
// in the sorted row order, and at gtab + gperm the token of every sorted row.
// A tile's X rows are gathered through it, its weight rows are its expert's
// rows of the stacked [E*n, k] weight, and its output rows are scattered back.
template <int F, int BM, int BN, int WGM, int WGN, int D, int UK, bool VEC, bool ROT, int SCHED, int DX, bool TS,
          bool GRP = false>
__global__ void __launch_bounds__(WGM *WGN * 64)
mfma_kernel(const uint8_t *__restrict__ codes, const void *__restrict__ scales, const uint16_t *__restrict__ biases,
            float global, const uint16_t *__restrict__ x, void *__restrict__ out, int ot, int64_t m, int64_t n,
            int64_t k, int tiles_m, int tiles_n, const int32_t *__restrict__ gtab, int64_t gperm) {
  constexpr int NTHR = WGM * WGN * 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MT = WTM / 32, NT = WTN / 32;
  constexpr int XCH = BM * (BK / 8) / NTHR;  // 16-byte X chunks per thread per step
  static_assert(XCH * NTHR == BM * (BK / 8), "X tile must split evenly");
  // X staging buffers: two, or three for the step-ahead schedule (SCHED 5)
  constexpr int NBX = SCHED == 5 ? 3 : 2;
  // int8 fold (step-ahead schedule; the small-problem schedule keeps hi + lo)
  constexpr bool FOLD = kFold<F> && SCHED == 5;
  constexpr bool SPLIT = kSplit<F> && !FOLD;
  // int8 fold: slice t, lane half h covers k = 32(t/2) + 16h + 8(t%2) + 0..7, so
  // slices 0,1 hold block 2kt and slices 2,3 block 2kt+1 (each MFMA one block)
  constexpr bool P2 = FOLD && Traits<F>::kBits == 8;
  // one LDS array: the X buffers, reused by the epilogue's staging
  constexpr int XSZ = NBX * BM * LDS_LD, STG = epi::stage_bytes<WTN, WGM * WGN>() / 2;
  __shared__ __attribute__((aligned(16))) uint16_t smem[XSZ > STG ? XSZ : STG];
  auto xs = reinterpret_cast<uint16_t (*)[BM * LDS_LD]>(smem);

  // ---- tile mapping: contiguous tile runs per XCD ----
  const int T = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((T & 7) == 0) t = (t & 7) * (T >> 3) + (t >> 3);
  const int tm = t / tiles_n, tn = t - tm * tiles_n;
  int64_t m0 = (int64_t)tm * BM, mlim = m, wrow0 = 0;  // first row, row limit, first weight row
  const int32_t *perm = nullptr;
  if constexpr (GRP) {
    if (tm >= gtab[0]) return;  // uniform: a tile past those the routing produced
    const int32_t *tile = gtab + 1 + 3 * tm;
    wrow0 = (int64_t)tile[0] * n;
    m0 = tile[1];
    mlim = tile[2];
    perm = gtab + gperm;
  }
  const int64_t n0 = (int64_t)tn * BN;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid - (wid / WGN) * WGN;
  const int l32 = lane & 31, h = lane >> 5;

  // X chunk c of this thread: tile row cid / 8, 8-element column group cid % 8.
  const uint16_t *xp[XCH];
#pragma unroll
  for (int c = 0; c < XCH; ++c) {
    const int cid = c * NTHR + tid;
    const int64_t gr = m0 + (cid >> 3);
    const int64_t row = gr < mlim ? gr : mlim - 1;  // rows past the limit read a valid row; never stored
    xp[c] = x + (GRP ? (int64_t)perm[row] : row) * k + (cid & 7) * 8;
  }
  int64_t wcol[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int64_t gc = n0 + wn * WTN + j * 32 + l32;
    wcol[j] = wrow0 + (gc < n ? gc : n - 1);
  }

  f32x16_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int KT = (int)((k + BK - 1) / BK);  // k steps, the last one possibly ragged
  const int KF = (int)(k / BK);              // full k steps
  // Rotation of the k walk: the workgroups that run together on one XCD start
  // at different k steps, so their concurrent requests spread over the L2
  // channels instead of all hitting the same rows' lines at once.  Only when
  // every step is full (the sum is order-free up to fp32 rounding).
  int krot = 0;
  if (ROT && KF == KT) krot = (int)(((int64_t)(blockIdx.x >> 3) * 7) % KT);
  Slot<XCH, NT> G[D];

  // Loads of step kt into a slot; GUARD handles the ragged last step.
  auto load = [&](auto guard, Slot<XCH, NT> &g, int kt) {
    constexpr bool kGuard = decltype(guard)::value;
    if (ROT) {
      kt += krot;
      if (kt >= KT) kt -= KT;
    }
    const int64_t k0 = (int64_t)kt * BK;
    const bool tail = kGuard && kt >= KF;
#pragma unroll
    for (int c = 0; c < XCH; ++c) {
      if (!kGuard || !tail || k0 + ((c * NTHR + tid) & 7) * 8 < k)
        g.x[c] = *reinterpret_cast<const uint4 *>(xp[c] + k0);
      else
        g.x[c] = make_uint4(0, 0, 0, 0);
    }
    const int64_t kb = k0 + 32 * h;
#pragma unroll
    for (int j = 0; j < NT; ++j) load_w<F, VEC>(g.w[j], codes, scales, biases, wcol[j], k, kb, tail);
  };
  auto store_x = [&](const Slot<XCH, NT> &g, int buf) {
#pragma unroll
    for (int c = 0; c < XCH; ++c) {
      const int cid = c * NTHR + tid;
      *reinterpret_cast<uint4 *>(&xs[buf][(cid >> 3) * LDS_LD + (cid & 7) * 8]) = g.x[c];
    }
  };
  // One k step: decode this step's weights, refill the slot with step kt + D,
  // multiply from LDS, stage step kt + 1 into the other LDS buffer.
  auto read_a = [&](const uint16_t *xb, int s, bf16x8_t a[MT]) {
    const int ko = P2 ? 32 * (s >> 1) + 16 * h + 8 * (s & 1) : 32 * h + 8 * s;
#pragma unroll
    for (int i = 0; i < MT; ++i)
      a[i] = *reinterpret_cast<const bf16x8_t *>(&xb[(wm * WTM + i * 32 + l32) * LDS_LD + ko]);
  };
  auto mma = [&](const bf16x8_t a[MT], const bf16x8_t bh[NT], const bf16x8_t bl[NT]) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bh[j], acc[i][j], 0, 0, 0);
        if constexpr (SPLIT) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bl[j], acc[i][j], 0, 0, 0);
      }
  };
  auto step = [&](auto guard, int kt, Slot<XCH, NT> &cur, const Slot<XCH, NT> &nxt) {
    constexpr bool kGuard = decltype(guard)::value;
    const uint16_t *xb = xs[kt & 1];
    bf16x8_t bh[NT][4], bl[NT][4];
    if constexpr (SCHED == 4) {
      // Software-pipelined step in fenced phases: the MFMAs of slice s issue
      // alongside the LDS reads of slice s+1, the weight decode, the global
      // prefetch and (last) the LDS writes of the next step.
      bf16x8_t a0[MT], a1[MT];
      read_a(xb, 0, a0);
#pragma unroll
      for (int j = 0; j < NT; ++j) decode_w<F>(cur.w[j], bh[j], bl[j]);
      __builtin_amdgcn_sched_barrier(0);
      bf16x8_t bs[NT], ls[NT];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8_t *ac = (s & 1) ? a1 : a0;
        bf16x8_t *an = (s & 1) ? a0 : a1;
        if (s < 3) read_a(xb, s + 1, an);
        if (s == 1) {
          if (!kGuard || kt + D < KT) load(guard, cur, kt + D);
        }
        if (s == 3) {
          if (!kGuard || kt + 1 < KT) store_x(nxt, (kt + 1) & 1);
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          bs[j] = bh[j][s];
          ls[j] = bl[j][s];
        }
        mma(ac, bs, ls);
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
      return;
    }
    bf16x8_t af[4][MT];
    if constexpr (SCHED == 1) {
      // All A fragments of the step first: their LDS latency overlaps the
      // weight decode instead of stalling each MFMA pair.
#pragma unroll
      for (int s = 0; s < 4; ++s) read_a(xb, s, af[s]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) decode_w<F>(cur.w[j], bh[j], bl[j]);
    if (!kGuard || kt + D < KT) load(guard, cur, kt + D);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if constexpr (SCHED != 1) read_a(xb, s, af[s]);
      bf16x8_t bs[NT], ls[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        bs[j] = bh[j][s];
        ls[j] = bl[j][s];
      }
      mma(af[s], bs, ls);
    }
    if constexpr (SCHED == 2) __builtin_amdgcn_iglp_opt(0);
    if constexpr (SCHED == 3) __builtin_amdgcn_iglp_opt(1);
    if (!kGuard || kt + 1 < KT) store_x(nxt, (kt + 1) & 1);
    __syncthreads();
  };
  constexpr std::integral_constant<bool, false> kFast{};
  constexpr std::integral_constant<bool, true> kGuarded{};

  if constexpr (SCHED == 5) {
    // Step-ahead schedule.  Three X buffers: while step kt runs from buffer
    // kt%3, step kt+1 is already complete in (kt+1)%3 (its first A fragments
    // are read during step kt's last slice) and step kt+2 is written into
    // (kt+2)%3 at the end of step kt.  Weights stay in registers: step kt+1's
    // are decoded during step kt.  Rings: X of step kt+2 in one slot (loaded
    // a step ahead of its LDS write); W of steps kt+1 .. kt+D, step q in slot
    // q % D.  So the MFMA stream never waits on the barrier for its first
    // operands, only on the issue of its own slices.
    struct SX {
      uint4 x[XCH];
    };
    SX gx[DX];
    WRaw gw[D][NT];
    // trip scales (k % 256 == 0): words of the trip being decoded and of the
    // next one; step kt decodes step kt+1, so the switch to the next trip
    // happens in the last step of a trip, which then loads the trip after
    constexpr bool kTS = TS && kTripSc<F>;
    static_assert(!kTS || (UK == 4 && !ROT), "trip scales need 4-step trips and no rotation");
    uint32_t tsc[NT][kTripWords<F>], tsn[NT][kTripWords<F>];
    const int NTRIP = KT / 4;
    bf16x8_t a0[MT];                       // slice-0 A fragments of the current step
    bf16x8_t bh[NT][4], bl[NT][4];         // decoded B fragments of the current step
    float fs[NT][2], fsn[NT][2];           // fold factors of the current and next step (FOLD)
    f32x16_t pacc[MT][NT];                 // per-block partial sums (FOLD)
    const f32x16_t kZero = {};
    auto loadx = [&](auto guard, SX &g, int kt) {
      constexpr bool kG = decltype(guard)::value;
      if (ROT) {
        kt += krot;
        if (kt >= KT) kt -= KT;
      }
      const int64_t k0 = (int64_t)kt * BK;
      const bool tail = kG && kt >= KF;
#pragma unroll
      for (int c = 0; c < XCH; ++c) {
        if (!kG || !tail || k0 + ((c * NTHR + tid) & 7) * 8 < k) g.x[c] = *reinterpret_cast<const uint4 *>(xp[c] + k0);
        else g.x[c] = make_uint4(0, 0, 0, 0);
      }
    };
    auto loadw = [&](auto guard, WRaw (&w)[NT], int kt) {
      constexpr bool kG = decltype(guard)::value;
      if (ROT) {
        kt += krot;
        if (kt >= KT) kt -= KT;
      }
      const int64_t kb = (int64_t)kt * BK + (P2 ? 16 : 32) * h;
      const bool tail = kG && kt >= KF;
#pragma unroll
      for (int j = 0; j < NT; ++j) load_w<F, VEC, !kTS, P2>(w[j], codes, scales, biases, wcol[j], k, kb, tail);
    };
    auto loadsc = [&](uint32_t (&v)[NT][kTripWords<F>], int trip) {
#pragma unroll
      for (int j = 0; j < NT; ++j) load_trip_sc<F>(v[j], scales, biases, wcol[j], k, trip);
    };
    auto storex = [&](const SX &g, int buf) {
#pragma unroll
      for (int c = 0; c < XCH; ++c) {
        const int cid = c * NTHR + tid;
        *reinterpret_cast<uint4 *>(&xs[buf][(cid >> 3) * LDS_LD + (cid & 7) * 8]) = g.x[c];
      }
    };
    auto slice = [&](const bf16x8_t a[MT], auto SL) {
      constexpr int sl = decltype(SL)::value;
      if constexpr (FOLD) {
        constexpr bool first = P2 ? (sl & 1) == 0 : sl == 0;
        constexpr bool last = P2 ? (sl & 1) == 1 : sl == 3;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            if constexpr (first)
              pacc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bh[j][sl], kZero, 0, 0, 0);
            else
              pacc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bh[j][sl], pacc[i][j], 0, 0, 0);
            if constexpr (F == kINT4_AFFINE)  // bias * sum of the slice's x
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bl[j][0], acc[i][j], 0, 0, 0);
          }
        if constexpr (last) {
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j) {
              const float sc = P2 ? fs[j][sl >> 1] : fs[j][0];
#pragma unroll
              for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_fmaf(pacc[i][j][v], sc, acc[i][j][v]);
            }
        }
        return;
      }
      bf16x8_t bs[NT], ls[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        bs[j] = bh[j][sl];
        ls[j] = bl[j][sl];
      }
      mma(a, bs, ls);
    };
    auto step5 = [&](auto guard, int kt, WRaw (&wn)[NT], SX &xn, auto sidx) {
      constexpr bool kG = decltype(guard)::value;
      constexpr int SN = (decltype(sidx)::value + 1) % 4;  // step kt+1's place in its trip (kTS)
      const bool more = !kG || kt + 1 < KT;
      const uint16_t *xb = xs[kt % NBX];
      bf16x8_t a1[MT], bhn[NT][4], bln[NT][4];
      // slice 0: read slice 1
      read_a(xb, 1, a1);
      slice(a0, std::integral_constant<int, 0>{});
      __builtin_amdgcn_sched_barrier(0);
      // slice 1: read slice 2, decode the next step's weights (int8 fold: in
      // slice 2, where fewer registers are live than beside its first block fold)
      constexpr int kDec = FOLD ? 2 : 1;
      auto decode_next = [&]() {
        if (more) {
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            if constexpr (kTS) trip_sc<F, SN, FOLD>(wn[j], SN == 0 ? tsn[j] : tsc[j], h);
            decode_w<F, FOLD>(wn[j], bhn[j], bln[j], fsn[j]);
          }
        }
      };
      read_a(xb, 2, a0);
      if constexpr (kDec == 1) decode_next();
      slice(a1, std::integral_constant<int, 1>{});
      __builtin_amdgcn_sched_barrier(0);
      // slice 2: read slice 3, refill the weight slot with step kt+1+D (and,
      // when step kt+1 opened a trip, move to it and load the trip after)
      read_a(xb, 3, a1);
      if constexpr (kDec == 2) decode_next();
      if (!kG || kt + 1 + D < KT) loadw(guard, wn, kt + 1 + D);
      if constexpr (kTS && SN == 0) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int i = 0; i < kTripWords<F>; ++i) tsc[j][i] = tsn[j][i];
        if ((kt + 1) / 4 + 1 < NTRIP) loadsc(tsn, (kt + 1) / 4 + 1);
      }
      slice(a0, std::integral_constant<int, 2>{});
      __builtin_amdgcn_sched_barrier(0);
      // slice 3: read the next step's slice 0; after the MFMAs, X of step
      // kt+2 into its buffer and the X slot refilled with step kt+3
      if (more) read_a(xs[(kt + 1) % NBX], 0, a0);
      slice(a1, std::integral_constant<int, 3>{});
      if (!kG || kt + 2 < KT) {
        storex(xn, (kt + 2) % NBX);
        if (!kG || kt + 2 + DX < KT) loadx(guard, xn, kt + 2 + DX);
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          bh[j][t] = bhn[j][t];
          bl[j][t] = bln[j][t];
        }
        fs[j][0] = fsn[j][0];
        fs[j][1] = fsn[j][1];
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    };

    // prologue: steps 0 and 1 in LDS, step 2's X in its slot, step 0's
    // weights decoded, steps 1..D's weights in flight
    // every prologue load is issued before the first one is waited for
    {
      SX x1;
      WRaw w0[NT];
      loadx(kGuarded, gx[0], 0);
      if (KT > 1) loadx(kGuarded, x1, 1);
      if constexpr (kTS) {
        loadsc(tsc, 0);
        if (NTRIP > 1) loadsc(tsn, 1);
      }
      loadw(kGuarded, w0, 0);
#pragma unroll
      for (int q = 1; q <= D; ++q)
        if (q < KT) loadw(kGuarded, gw[q % D], q);
      storex(gx[0], 0);
      if (KT > 1) storex(x1, 1);
#pragma unroll
      for (int q = 2; q < 2 + DX; ++q)
        if (q < KT) loadx(kGuarded, gx[q % DX], q);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        if constexpr (kTS) trip_sc<F, 0, FOLD>(w0[j], tsc[j], h);
        decode_w<F, FOLD>(w0[j], bh[j], bl[j], fs[j]);
      }
    }
    __syncthreads();
    read_a(xs[0], 0, a0);

    static_assert(UK % D == 0 && UK % DX == 0, "UK must be a multiple of D and DX");
    constexpr int AHEAD = D + 1 > DX + 2 ? D + 1 : DX + 2;  // furthest step a steady step loads
    int kt = 0;
    for (; kt + UK + AHEAD <= KF; kt += UK) {
      Unroll<0, UK>::run([&](auto S) {
        constexpr int s_ = decltype(S)::value;
        step5(kFast, kt + s_, gw[(s_ + 1) % D], gx[(s_ + 2) % DX], S);
      });
    }
    // drain: kt stays a multiple of UK, so step kt + S uses the slots of S
    for (; kt < KT; kt += UK) {
      Unroll<0, UK>::run([&](auto S) {
        constexpr int s_ = decltype(S)::value;
        if (kt + s_ < KT) step5(kGuarded, kt + s_, gw[(s_ + 1) % D], gx[(s_ + 2) % DX], S);
      });
    }
  } else {

  // Prologue: steps 0..D-1 in flight, step 0 staged in LDS.
#pragma unroll
  for (int s = 0; s < D; ++s)
    if (s < KT) load(kGuarded, G[s], s);
  store_x(G[0], 0);
  __syncthreads();

  // Steady state: every step and every prefetch is a full step, no guards.
  // UK steps (a multiple of D) per trip: the compiler waits for all
  // outstanding loads at the loop back-edge, so that happens once per UK steps.
  static_assert(UK % D == 0, "UK must be a multiple of D");
  int kt = 0;
  for (; kt + UK + D <= KF; kt += UK) {
#pragma unroll
    for (int S = 0; S < UK; ++S) step(kFast, kt + S, G[S % D], G[(S + 1) % D]);
  }
  // Drain: the last steps, guarded.
  for (; kt < KT; kt += D) {
#pragma unroll
    for (int S = 0; S < D; ++S)
      if (kt + S < KT) step(kGuarded, kt + S, G[S], G[(S + 1) % D]);
  }

  }

  // ---- epilogue ----
  // epilogue: the X buffers are free now; each wave stages its tile there
  // (the nvfp4 global is applied here, once per output)
  __syncthreads();
  epi::store_acc<MT, NT, WTN>(acc, F == kNVFP4 ? global : 1.0f,
                              reinterpret_cast<uint8_t *>(smem) + wid * 32 * epi::row_stride<WTN, 4>(), lane,
                              m0 + wm * WTM, n0 + wn * WTN, mlim, n, out, ot, perm);
}

// Grouped launch: tiles_m is the most m-tiles the routing can produce, gtab /
// gperm the routing table (null for an ordinary launch).
struct Grp {
  const int32_t *gtab = nullptr;
  int64_t gperm = 0;
  int tiles_m = 0;
};

template <int F, int BM, int BN, int WGM, int WGN, int D, int UK, bool ROT = false, int SCHED = 1, int DX = 1>
hipError_t run_cfg(const QWeight &w, int64_t m, const void *x, void *out, int ot, hipStream_t s, const Grp &g = Grp()) {
  const int tiles_m = g.gtab ? g.tiles_m : (int)((m + BM - 1) / BM), tiles_n = (int)((w.n + BN - 1) / BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  const bool vec = Traits<F>::kBits == 8 || (w.k % 32) == 0;
  constexpr bool kTripOk = SCHED == 5 && UK == 4 && !ROT && kTripSc<F>;
  const dim3 block(WGM * WGN * 64);
  const auto *c = (const uint8_t *)w.codes;
  const auto *b = (const uint16_t *)w.biases;
  const auto *xx = (const uint16_t *)x;
  if (g.gtab) {  // grouped rows (k % 32 == 0 checked by the caller for 4-bit codes)
    if (kTripOk && w.k % 256 == 0)
      hipLaunchKernelGGL((mfma_kernel<F, BM, BN, WGM, WGN, D, UK, true, ROT, SCHED, DX, kTripOk, true>), grid, block, 0,
                         s, c, w.scales, b, w.global, xx, out, ot, m, w.n, w.k, tiles_m, tiles_n, g.gtab, g.gperm);
    else if (vec)
      hipLaunchKernelGGL((mfma_kernel<F, BM, BN, WGM, WGN, D, UK, true, ROT, SCHED, DX, false, true>), grid, block, 0,
                         s, c, w.scales, b, w.global, xx, out, ot, m, w.n, w.k, tiles_m, tiles_n, g.gtab, g.gperm);
    else
      return hipErrorInvalidValue;
  } else if (kTripOk && w.k % 256 == 0)
    hipLaunchKernelGGL((mfma_kernel<F, BM, BN, WGM, WGN, D, UK, true, ROT, SCHED, DX, kTripOk>), grid, block, 0, s, c,
                       w.scales, b, w.global, xx, out, ot, m, w.n, w.k, tiles_m, tiles_n, nullptr, 0);
  else if (vec)
    hipLaunchKernelGGL((mfma_kernel<F, BM, BN, WGM, WGN, D, UK, true, ROT, SCHED, DX, false>), grid, block, 0, s, c,
                       w.scales, b, w.global, xx, out, ot, m, w.n, w.k, tiles_m, tiles_n, nullptr, 0);
  else
    hipLaunchKernelGGL((mfma_kernel<F, BM, BN, WGM, WGN, D, UK, false, ROT, SCHED, DX, false>), grid, block, 0, s, c,
                       w.scales, b, w.global, xx, out, ot, m, w.n, w.k, tiles_m, tiles_n, nullptr, 0);
  return hipGetLastError();
}

template <int F>
hipError_t run_f(const QWeight &w, int64_t m, const void *x, void *out, int ot, hipStream_t s) {
  if ((m + 127) / 128 * ((w.n + 63) / 64) > (int64_t)1 << 30) return hipErrorInvalidValue;
  // Step-ahead schedule, 8 waves (two per SIMD), while the tiling gives at
  // least half a tile per CU: 128x256 tiles (one wave per 32 columns, all
  // 128 rows) first, as a 128-row X tile plus 256 weight columns is the
  // least global data per flop (measured at m=2048, n=k=4096: 63 vs 68 us for
  // 256x128; at m=512, n=11008, k=4096: 101-103 vs 106 us); then 256x128;
  // smaller problems use 128x64 tiles, ~3 workgroups per CU, and m <= 64
  // rows the 32- or 64-row tiles of the same schedule, so that the MFMAs do
  // not run 128 rows for a few (mxfp4 14336 x 4096, m = 16 / 64: 35.1 / 34.9
  // -> 22.2 / 27.9 us; int8 11008 x 4096, m = 16: 58.4 -> 38.5 us).  64-row
  // tiles also take over while the 128x64 grid would give at most half a
  // tile per CU (mxfp4 4096 x 4096, m = 96..256: 33.8-34.2 -> 26.3-27.3 us);
  // with more tiles than that, each extra m-tile's second decode of the
  // weight costs more than the fuller grid gains (mxfp4 14336 x 4096, m = 96:
  // 36.6 vs 47.0 us).
  const int64_t wide = ((m + 127) / 128) * ((w.n + 255) / 256);
  const int64_t tall = ((m + 255) / 256) * ((w.n + 127) / 128);
  const int64_t small = ((m + 127) / 128) * ((w.n + 63) / 64);
  if (w.n >= 256 && wide >= 128) return run_cfg<F, 128, 256, 1, 8, 1, 4, false, 5>(w, m, x, out, ot, s);
  if (tall >= 128) return run_cfg<F, 256, 128, 2, 4, 1, 4, false, 5>(w, m, x, out, ot, s);
  if (m <= 32) return run_cfg<F, 32, 64, 1, 2, 2, 4, false, 4>(w, m, x, out, ot, s);
  if (m <= 64 || small <= 128) return run_cfg<F, 64, 64, 2, 2, 2, 4, false, 4>(w, m, x, out, ot, s);
  return run_cfg<F, 128, 64, 2, 2, 2, 4, false, 4>(w, m, x, out, ot, s);
}

// Expert-grouped rows (the routing table from grouped.hip): 128-row tiles, so
// tiles never straddle two experts' rows; 128x256 tiles with the step-ahead
// schedule when the widest grid gives >= 128 tiles, else 128x64.  A grid of
// more than 256 wide tiles (one per CU) would leave a partly filled second
// round; there the formats whose 4-wave 128x128 kernel fits two workgroups
// per CU take that instead (1024 tokens top-2 of 8 mxfp4 experts of 4096 x
// 4096, 304 tiles of 128x256: 119 -> 112 us).
template <int F>
hipError_t run_grouped(const QWeight &w, int64_t m, const void *x, void *out, int ot, const int32_t *gtab,
                       int64_t gperm, int tiles_m, hipStream_t s) {
  const Grp g{gtab, gperm, tiles_m};
  if ((int64_t)tiles_m * ((w.n + 63) / 64) > (int64_t)1 << 30) return hipErrorInvalidValue;
  const int64_t wide = (int64_t)tiles_m * ((w.n + 255) / 256);
  if (!kFold<F> && w.n >= 256 && wide > 256)
    return run_cfg<F, 128, 128, 1, 4, 1, 4, false, 5>(w, m, x, out, ot, s, g);
  if (w.n >= 256 && wide >= 128) return run_cfg<F, 128, 256, 1, 8, 1, 4, false, 5>(w, m, x, out, ot, s, g);
  return run_cfg<F, 128, 64, 2, 2, 2, 4, false, 4>(w, m, x, out, ot, s, g);
}

}  // namespace

hipError_t launch_mfma_grouped(const QWeight &w, int64_t m, const void *x, void *out, int ot, const int32_t *gtab,
                               int64_t gperm, int tiles_m, hipStream_t s) {
  switch (w.fmt) {
    case kMXFP4: return run_grouped<kMXFP4>(w, m, x, out, ot, gtab, gperm, tiles_m, s);
    case kNVFP4: return run_grouped<kNVFP4>(w, m, x, out, ot, gtab, gperm, tiles_m, s);
    case kMXFP8_E4M3: return run_grouped<kMXFP8_E4M3>(w, m, x, out, ot, gtab, gperm, tiles_m, s);
    case kMXFP8_E5M2: return run_grouped<kMXFP8_E5M2>(w, m, x, out, ot, gtab, gperm, tiles_m, s);
    case kNVFP8: return run_grouped<kNVFP8>(w, m, x, out, ot, gtab, gperm, tiles_m, s);
    case kINT4_AFFINE: return run_grouped<kINT4_AFFINE>(w, m, x, out, ot, gtab, gperm, tiles_m, s);
    case kINT8_SYM: return run_grouped<kINT8_SYM>(w, m, x, out, ot, gtab, gperm, tiles_m, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mfma(const QWeight &w, int64_t m, const void *x, void *out, int ot, hipStream_t s) {
  switch (w.fmt) {
    case kMXFP4: return run_f<kMXFP4>(w, m, x, out, ot, s);
    case kNVFP4: return run_f<kNVFP4>(w, m, x, out, ot, s);
    case kMXFP8_E4M3: return run_f<kMXFP8_E4M3>(w, m, x, out, ot, s);
    case kMXFP8_E5M2: return run_f<kMXFP8_E5M2>(w, m, x, out, ot, s);
    case kNVFP8: return run_f<kNVFP8>(w, m, x, out, ot, s);
    case kINT4_AFFINE: return run_f<kINT4_AFFINE>(w, m, x, out, ot, s);
    case kINT8_SYM: return run_f<kINT8_SYM>(w, m, x, out, ot, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace bsq
