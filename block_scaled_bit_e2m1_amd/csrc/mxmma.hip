// mxmma.hip -- both-operands block-scaled GEMM on the gfx950 scaled MFMA:
//   out[i,j] = sum_p dequant(Xq)[i,p] * dequant(W)[j,p]
// with Xq and W both in an MX format (E2M1, E4M3 or E5M2 elements, one E8M0
// scale per 32 consecutive k).  This is the pages' TN scaled matmul: per
// block, acc += (a_scale * b_scale) * sum dec(a) * dec(b) [rlx-cpu quant.rs,
// lowp_scaled_matmul], which v_mfma_scale_f32_32x32x64_f8f6f4 executes in
// hardware: one instruction sums 64 k, i.e. two 32-element blocks, and the
// E8M0 scale of hardware block j comes from lane half j (lanes 32j..32j+31,
// one per row or column).  The instruction's k order differs by element width:
// a 4-bit operand lane of half h holds hardware k [32h, 32h+32); an 8-bit one
// holds [16h, 16h+16) in its bytes 0..15 and [32+16h, 48+16h) in bytes 16..31
// (both read off the instruction with one-hot inputs).
//
// k order.  A step covers 128 k = four 32-blocks = two MFMA slices; slice s
// puts logical block 2j+s in hardware block j, for both operands and either
// width, so lane half h always needs the scale bytes of blocks 2h and 2h+1
// (byte s selected by opsel) and the k orders of mixed-width pairs agree.
// In 16-byte chunks of a row's 64 (4-bit) or 128 (8-bit) code bytes per step,
// a 4-bit lane reads chunk 2h+s, an 8-bit lane chunks h+2s and 4+h+2s.
//
// Data movement.  Partial-line global loads leave the kernel bound by L1
// accesses, so every global load reads whole contiguous runs.  Both code
// tiles go from global memory straight into LDS (global_load_lds_dwordx4:
// a wave's 64 lanes fill 1 KB of LDS, lane l the 16 bytes at 16 l, with no
// registers in between), NB buffers deep, so the loads of a step are issued
// NB-1 steps before it runs.  Rows are stored with the 16-byte chunk index
// XOR-swizzled by row, the permutation applied on the global side (the lane
// that fills slot s of row r fetches the row's chunk s ^ key(r)), so that the
// per-lane operand reads are free of bank conflicts.  Scales are loaded once
// per 4 steps (16 bytes per row; four lanes per row, so their dword loads
// coalesce into one access), staged in LDS and read as one dword per row per
// step, one 4-step trip ahead; the steady loop is branch-free and the ragged
// end is a guarded drain.
//
// Geometry (CDNA4, wave64): workgroup tile 256x128 with 4x2 waves of 64x64
// (128x64 with 2x2 waves for small problems).  Tiles are renumbered so each
// XCD (own L2) runs a block of GM m-tiles by consecutive n-tiles, which
// bounds the W and X bytes one L2 must hold.
#include "bsq_internal.hpp"
#include "codec.hpp"
#include "epilogue.hpp"
#include "lds_swizzle.hpp"

#include <type_traits>

namespace bsq {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
// Register staging as native vectors (HIP's uint4 struct is copied with memcpy
// and kept in scratch memory).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BK = 128;  // k per step
constexpr int TRIP = 4;  // steps per scale load: 16 scale bytes per row

// scaled-MFMA operand format codes
template <int F> struct MxFmt;
template <> struct MxFmt<kMXFP8_E4M3> { static constexpr int kCode = 0, kBits = 8; };
template <> struct MxFmt<kMXFP8_E5M2> { static constexpr int kCode = 1, kBits = 8; };
template <> struct MxFmt<kMXFP4> { static constexpr int kCode = 4, kBits = 4; };

template <int FA, int FB, int BM, int BN, int WGM, int WGN, int NB, int GM>
__global__ void __launch_bounds__(WGM *WGN * 64)
mxmma_kernel(const uint8_t *__restrict__ xc, const uint8_t *__restrict__ xsc, const uint8_t *__restrict__ wc,
             const uint8_t *__restrict__ wsc, void *__restrict__ out, int ot, int64_t m, int64_t n, int64_t k,
             int tiles_m, int tiles_n) {
  constexpr int NTHR = WGM * WGN * 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MT = WTM / 32, NT = WTN / 32;
  constexpr int ABITS = MxFmt<FA>::kBits, BBITS = MxFmt<FB>::kBits;
  constexpr int XR = BK * ABITS / 8, WR = BK * BBITS / 8;  // code bytes per row per step
  constexpr int XCPR = XR / 16, WCPR = WR / 16;            // 16-byte chunks per row
  constexpr int NW = WGM * WGN;
  // the code tiles move in 1 KB blocks, one wave-wide 16-byte LDS-DMA load each
  constexpr int XBLK = BM * XR / 1024, WBLK = BN * WR / 1024;
  constexpr int LX = XBLK / NW, LW = WBLK / NW;  // blocks per wave per step
  constexpr int P = NB - 1;                      // steps the DMA loads run ahead
  constexpr int SCH = TRIP * (BM + BN) / NTHR;             // scale dwords per thread per trip
  constexpr int SCX = TRIP * BM / NTHR;                    // ... of which on X rows
  static_assert(LX * NW == XBLK && LW * NW == WBLK && LX > 0 && LW > 0, "code tiles must split into 1 KB blocks");
  static_assert(XCPR >= 1 && WCPR >= 1 && P >= 2, "whole chunks per row; at least two steps of lookahead");
  static_assert(SCH * NTHR == TRIP * (BM + BN) && SCX * NTHR == TRIP * BM, "scale tile must split evenly");
  static_assert(WTM % Swz<XR>::kPeriod == 0 && WTN % Swz<WR>::kPeriod == 0 && 32 % Swz<XR>::kPeriod == 0 &&
                    32 % Swz<WR>::kPeriod == 0,
                "one swizzle key per lane");
  // NB code buffers: step kt is read while step kt+1 is complete (so its
  // first fragments can be fetched early) and steps kt+2 .. kt+P are in flight
  // scales as [step of the trip][row], the step stride padded to 16 mod 64
  // words so that the writes (4 steps x 16 rows per pass) and the per-step
  // column reads both spread over all banks
  constexpr int SS = BM + BN + 16;
  constexpr int XB = BM * XR, WB = BN * WR;  // bytes of one code buffer
  // one LDS array: X buffers, W buffers, scale buffers (the epilogue reuses
  // the code buffers for staging)
  __shared__ __attribute__((aligned(16))) uint8_t smem[NB * (XB + WB) + 2 * TRIP * SS * 4];
  auto xs = [&](int b) __attribute__((always_inline)) { return smem + b * XB; };
  auto ws = [&](int b) __attribute__((always_inline)) { return smem + NB * XB + b * WB; };
  uint32_t(*ss)[TRIP * SS] = reinterpret_cast<uint32_t(*)[TRIP * SS]>(smem + NB * (XB + WB));

  // tile order: XCD x runs tiles [x*T/8, (x+1)*T/8) (blocks are dealt to the
  // XCDs round-robin), walked as GM m-tiles by consecutive n-tiles
  const int T = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((T & 7) == 0) t = (t & 7) * (T >> 3) + (t >> 3);
  const int grp = t / (GM * tiles_n), tin = t - grp * (GM * tiles_n);
  const int gm = min(GM, tiles_m - grp * GM);
  const int tm = grp * GM + tin % gm, tn = tin / gm;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid - (wid / WGN) * WGN;
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t nblk = k / 32;
  const int64_t xrb = k * ABITS / 8, wrb = k * BBITS / 8;  // code bytes per row
  const int KT = (int)(k / BK);

  // LDS-DMA sources: block c of this wave covers LDS bytes [1024 (wu + c NW),
  // + 1024) of a code buffer, lane l the 16 bytes at 16 l of it, i.e. slot s
  // of row r; the row's chunk that belongs there is s ^ key(r) (rows past m
  // or n read a valid row and are never stored)
  const int wu = __builtin_amdgcn_readfirstlane(wid);
  const uint8_t *xsrc[LX];
  const uint8_t *wsrc[LW];
#pragma unroll
  for (int c = 0; c < LX; ++c) {
    const int o = 1024 * (wu + c * NW) + 16 * lane, r = o / XR, s = (o % XR) >> 4;
    const int64_t gr = m0 + r;
    xsrc[c] = xc + (gr < m ? gr : m - 1) * xrb + ((s ^ Swz<XR>::key(r)) << 4);
  }
#pragma unroll
  for (int c = 0; c < LW; ++c) {
    const int o = 1024 * (wu + c * NW) + 16 * lane, r = o / WR, s = (o % WR) >> 4;
    const int64_t gr = n0 + r;
    wsrc[c] = wc + (gr < n ? gr : n - 1) * wrb + ((s ^ Swz<WR>::key(r)) << 4);
  }
  // scale dwords: item q = c*NTHR + tid is row q/TRIP (X rows, then W rows), step q%TRIP of a trip
  const uint8_t *sp[SCH];
  const int sst = tid % TRIP;
#pragma unroll
  for (int c = 0; c < SCH; ++c) {
    const int r = (c * NTHR + tid) / TRIP;
    if (c < SCX) {
      const int64_t gr = m0 + r;
      sp[c] = xsc + (gr < m ? gr : m - 1) * nblk;
    } else {
      const int64_t gr = n0 + (r - BM);
      sp[c] = wsc + (gr < n ? gr : n - 1) * nblk;
    }
  }
  // swizzle keys of this lane's operand rows (the same for all its rows)
  const int akey = Swz<XR>::key(l32), bkey = Swz<WR>::key(l32);
  const int ach0 = ((ABITS == 4 ? 2 * h : h) ^ akey) << 4, ach1 = ((ABITS == 4 ? 2 * h + 1 : h + 2) ^ akey) << 4;
  const int ahi0 = ((4 + h) ^ akey) << 4, ahi1 = ((6 + h) ^ akey) << 4;
  const int bch0 = ((BBITS == 4 ? 2 * h : h) ^ bkey) << 4, bch1 = ((BBITS == 4 ? 2 * h + 1 : h + 2) ^ bkey) << 4;
  const int bhi0 = ((4 + h) ^ bkey) << 4, bhi1 = ((6 + h) ^ bkey) << 4;
  const int arow = (wm * WTM + l32) * XR, brow = (wn * WTN + l32) * WR;
  const int asrow = wm * WTM + l32, bsrow = BM + wn * WTN + l32;
  const int sw = (tid / TRIP) + sst * SS;  // this thread's scale item 0 in the LDS layout

  f32x16_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  uint32_t R[SCH];  // scale dwords of the next trip

  // step kt's codes straight from global memory into code buffer kt % NB
  // (global_load_lds: no registers; counted by vmcnt until they land in LDS)
  // (the builtin's LDS pointer type exists only in the device pass)
  auto dma = [&](int kt) __attribute__((always_inline)) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int b = kt % NB;
#pragma unroll
    for (int c = 0; c < LX; ++c)
      __builtin_amdgcn_global_load_lds(xsrc[c] + (int64_t)kt * XR, smem + b * XB + 1024 * (wu + c * NW), 16, 0, 0);
#pragma unroll
    for (int c = 0; c < LW; ++c)
      __builtin_amdgcn_global_load_lds(wsrc[c] + (int64_t)kt * WR, smem + NB * XB + b * WB + 1024 * (wu + c * NW), 16,
                                       0, 0);
#endif
  };
  // scales of trip tr; steps past the end are clamped to the last one, so a
  // partial (or nonexistent) trip reads in bounds
  auto load_sc = [&](int tr) __attribute__((always_inline)) {
    const int st = min(tr * TRIP + sst, KT - 1);
#pragma unroll
    for (int c = 0; c < SCH; ++c) R[c] = *reinterpret_cast<const uint32_t *>(sp[c] + 4 * st);
  };
  auto store_sc = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < SCH; ++c) ss[buf][sw + c * (NTHR / TRIP)] = R[c];
  };

  // operand fragments of slice s from the LDS tiles of buffer buf
  auto read = [&](int buf, int s, i32x8_t a[MT], i32x8_t b[NT]) __attribute__((always_inline)) {
    const uint8_t *xb = xs(buf) + arow;
    const uint8_t *wb = ws(buf) + brow;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const uint8_t *row = xb + i * 32 * XR;
      const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(row + (s ? ach1 : ach0));
      const u32x4_t hi =
          ABITS == 8 ? *reinterpret_cast<const u32x4_t *>(row + (s ? ahi1 : ahi0)) : u32x4_t{0, 0, 0, 0};
      a[i] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint8_t *row = wb + j * 32 * WR;
      const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(row + (s ? bch1 : bch0));
      const u32x4_t hi =
          BBITS == 8 ? *reinterpret_cast<const u32x4_t *>(row + (s ? bhi1 : bhi0)) : u32x4_t{0, 0, 0, 0};
      b[j] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  };
  // the 2x MT x NT MFMAs of slice s; the scale operand's byte s is this lane's E8M0 for slice s
  auto mma = [&](auto sl, const i32x8_t a[MT], const i32x8_t b[NT], const uint32_t as[MT], const uint32_t bs[NT])
                 __attribute__((always_inline)) {
    constexpr int s = decltype(sl)::value;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], MxFmt<FA>::kCode,
                                                                   MxFmt<FB>::kCode, s, (int)as[i], s, (int)bs[j]);
  };
  constexpr std::integral_constant<int, 0> kS0{};
  constexpr std::integral_constant<int, 1> kS1{};
  // scale bytes of step kt for this lane's rows: blocks 4kt+2h and 4kt+2h+1 in bytes 0 and 1
  auto read_sc = [&](int kt, uint32_t as[MT], uint32_t bs[NT]) __attribute__((always_inline)) {
    const uint32_t *sb = ss[(kt / TRIP) & 1] + (kt % TRIP) * SS;
#pragma unroll
    for (int i = 0; i < MT; ++i) as[i] = sb[asrow + i * 32] >> (16 * h);
#pragma unroll
    for (int j = 0; j < NT; ++j) bs[j] = sb[bsrow + j * 32] >> (16 * h);
  };

  // loop-carried: slice-0 fragments and scale bytes of the current step
  i32x8_t a0[MT], b0[NT];
  uint32_t as[MT], bs[NT];

  // The step-end barrier: each wave waits until at most N of its vector
  // memory operations are outstanding (loads complete in issue order, so the
  // DMA loads of the step read next are in LDS), for its LDS operations, then
  // meets the others.  Written out because __syncthreads' release fence
  // would wait for every DMA load in flight, i.e. drain the lookahead.
  auto bar = [&](auto Nc) __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(decltype(Nc)::value) : "memory");
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // Vector memory operations a steady step kt issues after the DMA loads of
  // step kt+2: the DMA loads of steps kt+3 .. kt+P, and the scale loads of
  // the steps kt+2-P .. kt that fetch a trip (step index TRIP-2 in a trip,
  // after that step's DMA loads).
  auto after = [](int S) constexpr {
    int nsc = 0;
    for (int d = 0; d <= P - 2; ++d)
      if ((((S - d) % TRIP) + TRIP) % TRIP == TRIP - 2) ++nsc;
    return (P - 2) * (LX + LW) + nsc * SCH;
  };

  // One step kt (S = kt % TRIP).  Code buffer kt%NB holds step kt and
  // (kt+1)%NB step kt+1 (complete since the last barrier); steps kt+2 ..
  // kt+P-1 are on their way.  The step issues the DMA loads of step kt+P
  // into buffer (kt+P)%NB, whose last reader (step kt-1) has passed the
  // barrier.
  auto step = [&](auto guard, int kt, auto Sc) __attribute__((always_inline)) {
    constexpr bool kGuard = decltype(guard)::value;
    constexpr int S = decltype(Sc)::value;  // kt % TRIP (steady steps only)
    const int s_ = kGuard ? kt % TRIP : S;
    const bool more = !kGuard || kt + 1 < KT;
    i32x8_t a1[MT], b1[NT];
    uint32_t asn[MT], bsn[NT];
    // phase 1: slice-1 fragments go out, then the slice-0 MFMAs on operands
    // fetched during the previous step
    read(kt % NB, 1, a1, b1);
    mma(kS0, a0, b0, as, bs);
    __builtin_amdgcn_sched_barrier(0);
    // phase 2: the next step's slice-0 fragments and scales, the slice-1
    // MFMAs, then the DMA loads of step kt+P
    if (more) {
      read((kt + 1) % NB, 0, a0, b0);
      read_sc(kt + 1, asn, bsn);
    }
    mma(kS1, a1, b1, as, bs);
    if (!kGuard || kt + P < KT) dma(kt + P);
    if (s_ == TRIP - 2 && more) {
      // publish the next trip's scales one step early (the last step of this
      // trip reads them ahead), fetch the trip after
      store_sc(((kt / TRIP) + 1) & 1);
      load_sc(kt / TRIP + 2);
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) as[i] = asn[i];
#pragma unroll
    for (int j = 0; j < NT; ++j) bs[j] = bsn[j];
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kGuard) bar(std::integral_constant<int, 0>{});
    else bar(std::integral_constant<int, after(S)>{});
  };
  constexpr std::integral_constant<bool, false> kFast{};
  constexpr std::integral_constant<bool, true> kGuarded{};

  // prologue: trip-0 scales in LDS, the DMA loads of steps 0 .. P-1 issued
  // together and all waited for
  load_sc(0);
#pragma unroll
  for (int q = 0; q < P; ++q)
    if (q < KT) dma(q);
  store_sc(0);
  load_sc(1);
  bar(std::integral_constant<int, 0>{});
  read(0, 0, a0, b0);
  read_sc(0, as, bs);
  int kt = 0;
  // steady state: whole trips whose loads, writes and reads all stay in range
  for (; kt + TRIP + P <= KT; kt += TRIP) {
    step(kFast, kt + 0, std::integral_constant<int, 0>{});
    step(kFast, kt + 1, std::integral_constant<int, 1>{});
    step(kFast, kt + 2, std::integral_constant<int, 2>{});
    step(kFast, kt + 3, std::integral_constant<int, 3>{});
  }
  static_assert(TRIP == 4, "the steady loop is written out for 4-step trips");
  // guarded drain: every step waits for all its loads
  for (; kt < KT; ++kt) step(kGuarded, kt, std::integral_constant<int, 0>{});

  // epilogue: the code buffers are free now; each wave stages its tile there
  static_assert(epi::stage_bytes<WTN, WGM * WGN>() <= NB * (XB + WB), "staging must fit in the code buffers");
  __syncthreads();
  epi::store_acc<MT, NT, WTN>(acc, 1.0f, smem + wid * 32 * epi::row_stride<WTN, 4>(), lane, m0 + wm * WTM,
                              n0 + wn * WTN, m, n, out, ot);
}

template <int FA, int FB, int BM, int BN, int NB, int GM, int WGM = 2, int WGN = 2>
hipError_t run_cfg(const void *xc, const void *xs, const void *wc, const void *ws, int64_t m, int64_t n, int64_t k,
                   void *out, int ot, hipStream_t s) {
  const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + BN - 1) / BN);
  hipLaunchKernelGGL((mxmma_kernel<FA, FB, BM, BN, WGM, WGN, NB, GM>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(WGM * WGN * 64), 0,
                     s, (const uint8_t *)xc, (const uint8_t *)xs, (const uint8_t *)wc, (const uint8_t *)ws, out, ot, m,
                     n, k, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int FA, int FB>
hipError_t run_ab(const void *xc, const void *xs, const void *wc, const void *ws, int64_t m, int64_t n, int64_t k,
                  void *out, int ot, hipStream_t s) {
  if ((m + 127) / 128 * ((n + 63) / 64) > (int64_t)1 << 30) return hipErrorInvalidValue;
  const int64_t big = ((m + 255) / 256) * ((n + 127) / 128);
  // Measured on 2048x4096x4096 (us, fp4 x fp4 / e4m3 x e4m3): codes through
  // registers with one step of prefetch 33.9 / 52.2; LDS-DMA loads 32.4 /
  // 50.9; and 4x2 waves of 64x64 instead of 2x4 of 128x32 (fp4) and 2x2 of
  // 128x64 (8-bit pairs; a quarter less LDS operand traffic per MFMA) 31.8 /
  // 47.4.  NB: 4 code buffers when one step's tiles take at most 32 KB, else
  // 3 (LDS: 160 KB per CU).
  constexpr int A8 = MxFmt<FA>::kBits == 8, B8 = MxFmt<FB>::kBits == 8;
  if (big >= 256) {
    if constexpr (A8 && B8) return run_cfg<FA, FB, 256, 128, 3, 4, 4, 2>(xc, xs, wc, ws, m, n, k, out, ot, s);
    else if constexpr (A8) return run_cfg<FA, FB, 256, 128, 3, 4, 4, 2>(xc, xs, wc, ws, m, n, k, out, ot, s);
    else if constexpr (B8) return run_cfg<FA, FB, 256, 128, 4, 4, 4, 2>(xc, xs, wc, ws, m, n, k, out, ot, s);
    else return run_cfg<FA, FB, 256, 128, 4, 4, 4, 2>(xc, xs, wc, ws, m, n, k, out, ot, s);
  }
  return run_cfg<FA, FB, 128, 64, 3, 4, 2, 2>(xc, xs, wc, ws, m, n, k, out, ot, s);
}

template <int FA>
hipError_t run_a(int wfmt, const void *xc, const void *xs, const void *wc, const void *ws, int64_t m, int64_t n,
                 int64_t k, void *out, int ot, hipStream_t s) {
  switch (wfmt) {
    case kMXFP4: return run_ab<FA, kMXFP4>(xc, xs, wc, ws, m, n, k, out, ot, s);
    case kMXFP8_E4M3: return run_ab<FA, kMXFP8_E4M3>(xc, xs, wc, ws, m, n, k, out, ot, s);
    case kMXFP8_E5M2: return run_ab<FA, kMXFP8_E5M2>(xc, xs, wc, ws, m, n, k, out, ot, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_mxmma(int xfmt, const void *xc, const void *xs, int wfmt, const void *wc, const void *ws, int64_t m,
                        int64_t n, int64_t k, void *out, int ot, hipStream_t s) {
  switch (xfmt) {
    case kMXFP4: return run_a<kMXFP4>(wfmt, xc, xs, wc, ws, m, n, k, out, ot, s);
    case kMXFP8_E4M3: return run_a<kMXFP8_E4M3>(wfmt, xc, xs, wc, ws, m, n, k, out, ot, s);
    case kMXFP8_E5M2: return run_a<kMXFP8_E5M2>(wfmt, xc, xs, wc, ws, m, n, k, out, ot, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace bsq
