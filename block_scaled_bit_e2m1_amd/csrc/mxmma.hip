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
// Geometry (CDNA4, wave64): workgroup tile 256x128, 2x2 waves (wave tile
// 128x64), k step 128 = four 32-blocks = two MFMA slices.  Slice s puts
// logical block 2j+s in hardware block j, for both operands and either width,
// so lane half h always owns the scale pair of blocks 2h, 2h+1 (one 16-bit
// load, byte s selected by opsel) and the k orders of mixed-width pairs agree:
// 4-bit lanes read the 64 contiguous codes of blocks 2h, 2h+1 (32 bytes),
// 8-bit lanes the 16-byte pieces at 16h + 32q, q = 0..3 (slice s uses q = s
// and q = 2+s).  W codes go straight from HBM into B-operand registers; X
// codes are staged through LDS (double buffered, rows padded to 144 B) and
// their scales loaded like W's.  Two-deep register prefetch, branch-free
// steady state (4 steps per loop trip), XCD-aware tile order, as in the bf16
// MFMA kernel.
#include "bsq_internal.hpp"
#include "codec.hpp"

#include <type_traits>

namespace bsq {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
// Slot data as a native vector (HIP's uint4 struct is copied with memcpy and
// kept in scratch memory).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BKX = 128;          // k per step
constexpr int LDX = BKX + 16;     // bytes per LDS row of the X code tile (8-bit codes)

// scaled-MFMA operand format codes
template <int F> struct MxFmt;
template <> struct MxFmt<kMXFP8_E4M3> { static constexpr int kCode = 0, kBits = 8; };
template <> struct MxFmt<kMXFP8_E5M2> { static constexpr int kCode = 1, kBits = 8; };
template <> struct MxFmt<kMXFP4> { static constexpr int kCode = 4, kBits = 4; };

// One lane's data for one step: its codes (32 bytes for 4-bit, four 16-byte
// pieces for 8-bit) and the E8M0 scale bytes of blocks 2h and 2h+1.
template <int FB>
struct WSlot {
  u32x4_t c[MxFmt<FB>::kBits / 2];  // 2 (4-bit) or 4 (8-bit) x 16 bytes
  uint32_t s;                     // two scale bytes (low byte: first 32-block)
};

template <int FA, int FB, int BM, int BN, int WGM, int WGN, int D, int UK>
__global__ void __launch_bounds__(WGM *WGN * 64)
mxmma_kernel(const uint8_t *__restrict__ xc, const uint8_t *__restrict__ xsc, const uint8_t *__restrict__ wc,
             const uint8_t *__restrict__ wsc, void *__restrict__ out, int ot, int64_t m, int64_t n, int64_t k,
             int tiles_m, int tiles_n) {
  constexpr int NTHR = WGM * WGN * 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MT = WTM / 32, NT = WTN / 32;
  constexpr int ABITS = MxFmt<FA>::kBits, BBITS = MxFmt<FB>::kBits;
  constexpr int XROW = BKX * ABITS / 8;          // bytes of X codes per row per step (128 or 64)
  constexpr int XCH = BM * (XROW / 16) / NTHR;   // 16-byte X chunks per thread per step
  constexpr int CPR = XROW / 16;                 // chunks per row
  static_assert(XCH * NTHR == BM * CPR, "X tile must split evenly");
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][BM * LDX];

  const int T = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((T & 7) == 0) t = (t & 7) * (T >> 3) + (t >> 3);
  const int tm = t / tiles_n, tn = t - tm * tiles_n;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid - (wid / WGN) * WGN;
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t nblk = k / 32;
  const int64_t xrb = k * ABITS / 8, wrb = k * BBITS / 8;  // code bytes per row

  const uint8_t *xp[XCH];
#pragma unroll
  for (int c = 0; c < XCH; ++c) {
    const int cid = c * NTHR + tid;
    const int64_t gr = m0 + cid / CPR;
    xp[c] = xc + (gr < m ? gr : m - 1) * xrb + (cid % CPR) * 16;  // rows past m: valid, never stored
  }
  const uint8_t *wp[NT];
  const uint8_t *wsp[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    int64_t gc = n0 + wn * WTN + j * 32 + l32;
    gc = gc < n ? gc : n - 1;
    wp[j] = wc + gc * wrb + (BBITS == 4 ? 32 : 16) * h;
    wsp[j] = wsc + gc * nblk + 2 * h;
  }
  const uint8_t *xsp[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    int64_t gr = m0 + wm * WTM + i * 32 + l32;
    gr = gr < m ? gr : m - 1;
    xsp[i] = xsc + gr * nblk + 2 * h;
  }

  f32x16_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int KT = (int)(k / BKX);
  struct Slot {
    u32x4_t x[XCH];
    WSlot<FB> w[NT];
    uint32_t xs2[MT];  // X scale byte pairs of this lane's rows
  };
  Slot G[D];

  auto load = [&](Slot &g, int kt) __attribute__((always_inline)) {
    const int64_t k0 = (int64_t)kt * BKX;
#pragma unroll
    for (int c = 0; c < XCH; ++c) g.x[c] = *reinterpret_cast<const u32x4_t *>(xp[c] + k0 * ABITS / 8);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int q = 0; q < BBITS / 2; ++q)
        g.w[j].c[q] = *reinterpret_cast<const u32x4_t *>(wp[j] + k0 * BBITS / 8 + (BBITS == 4 ? 16 : 32) * q);
      g.w[j].s = *reinterpret_cast<const uint16_t *>(wsp[j] + k0 / 32);
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) g.xs2[i] = *reinterpret_cast<const uint16_t *>(xsp[i] + k0 / 32);
  };
  auto store_x = [&](const Slot &g, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < XCH; ++c) {
      const int cid = c * NTHR + tid;
      *reinterpret_cast<u32x4_t *>(&xs[buf][(cid / CPR) * LDX + (cid % CPR) * 16]) = g.x[c];
    }
  };
  auto step = [&](auto guard, int kt, Slot &cur, const Slot &nxt) __attribute__((always_inline)) {
    constexpr bool kGuard = decltype(guard)::value;
    const uint8_t *xb = xs[kt & 1];
    // A operands of both slices: 16 (4-bit) or 2 x 16 (8-bit) bytes per lane each
    i32x8_t a[2][MT];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const uint8_t *row = &xb[(wm * WTM + i * 32 + l32) * LDX];
        const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(row + (ABITS == 4 ? 32 * h + 16 * s : 16 * h + 32 * s));
        const u32x4_t hi = ABITS == 8 ? *reinterpret_cast<const u32x4_t *>(row + 64 + 16 * h + 32 * s) : u32x4_t{0, 0, 0, 0};
        a[s][i] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    i32x8_t b[2][NT];
    uint32_t bs[NT], as[MT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      bs[j] = cur.w[j].s;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if constexpr (BBITS == 4) {
          const u32x4_t c = cur.w[j].c[s];
          b[s][j] = i32x8_t{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
        } else {
          const u32x4_t c0 = cur.w[j].c[s], c1 = cur.w[j].c[2 + s];
          b[s][j] = i32x8_t{(int)c0.x, (int)c0.y, (int)c0.z, (int)c0.w, (int)c1.x, (int)c1.y, (int)c1.z, (int)c1.w};
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) as[i] = cur.xs2[i];
    __builtin_amdgcn_sched_barrier(0);
    if (!kGuard || kt + D < KT) load(cur, kt + D);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          // the scale operand's byte s is this lane's E8M0 for slice s
          if (s == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[0][i], b[0][j], acc[i][j], MxFmt<FA>::kCode,
                                                                       MxFmt<FB>::kCode, 0, (int)as[i], 0, (int)bs[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[1][i], b[1][j], acc[i][j], MxFmt<FA>::kCode,
                                                                       MxFmt<FB>::kCode, 1, (int)as[i], 1, (int)bs[j]);
        }
    if (!kGuard || kt + 1 < KT) store_x(nxt, (kt + 1) & 1);
    __syncthreads();
  };
  constexpr std::integral_constant<bool, false> kFast{};
  constexpr std::integral_constant<bool, true> kGuarded{};

#pragma unroll
  for (int s = 0; s < D; ++s)
    if (s < KT) load(G[s], s);
  store_x(G[0], 0);
  __syncthreads();
  int kt = 0;
  for (; kt + UK + D <= KT; kt += UK) {
#pragma unroll
    for (int S = 0; S < UK; ++S) step(kFast, kt + S, G[S % D], G[(S + 1) % D]);
  }
  for (; kt < KT; kt += D) {
#pragma unroll
    for (int S = 0; S < D; ++S)
      if (kt + S < KT) step(kGuarded, kt + S, G[S], G[(S + 1) % D]);
  }

#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int64_t col = n0 + wn * WTN + j * 32 + l32;
      if (col >= n) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * WTM + i * 32 + (v >> 2) * 8 + h * 4 + (v & 3);
        if (row >= m) continue;
        const float val = acc[i][j][v];
        if (ot == 0) reinterpret_cast<float *>(out)[row * n + col] = val;
        else reinterpret_cast<uint16_t *>(out)[row * n + col] = f32_to_bf16_bits(val);
      }
    }
  }
}

template <int FA, int FB, int BM, int BN>
hipError_t run_cfg(const void *xc, const void *xs, const void *wc, const void *ws, int64_t m, int64_t n, int64_t k,
                   void *out, int ot, hipStream_t s) {
  const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + BN - 1) / BN);
  hipLaunchKernelGGL((mxmma_kernel<FA, FB, BM, BN, 2, 2, 2, 4>), dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, s,
                     (const uint8_t *)xc, (const uint8_t *)xs, (const uint8_t *)wc, (const uint8_t *)ws, out, ot, m, n,
                     k, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int FA, int FB>
hipError_t run_ab(const void *xc, const void *xs, const void *wc, const void *ws, int64_t m, int64_t n, int64_t k,
                  void *out, int ot, hipStream_t s) {
  if ((m + 127) / 128 * ((n + 63) / 64) > (int64_t)1 << 30) return hipErrorInvalidValue;
  const int64_t big = ((m + 255) / 256) * ((n + 127) / 128);
  if (big >= 256) return run_cfg<FA, FB, 256, 128>(xc, xs, wc, ws, m, n, k, out, ot, s);
  return run_cfg<FA, FB, 128, 64>(xc, xs, wc, ws, m, n, k, out, ot, s);
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
