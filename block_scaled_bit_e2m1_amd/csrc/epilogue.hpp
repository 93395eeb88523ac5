// epilogue.hpp -- writes a wave's fp32 accumulator tiles of a 32x32 MFMA
// (lane l holds column l%32, rows 8(v/4) + 4(l/32) + v%4 of each tile, v =
// 0..15) to a row-major [m, n] output, f32 or bf16 (round to nearest even).
//
// Stored directly, each lane would write 2- or 4-byte pieces of one column.
// Instead every 32-row band of the wave tile is staged in LDS and read back
// as 16-byte row pieces, so one store instruction writes whole row runs of
// the tile; pieces that cross the right edge of the output, or outputs whose
// rows are not 16-byte aligned, are written element by element.  The 16-byte
// stores are nontemporal: every workgroup writes its whole tile at the end,
// so the output is a burst of writes nothing reads back soon (measured on
// 2048x4096 bf16 outputs: 1-2 us less per GEMM).  The caller
// passes an LDS region nobody else uses during the call (the kernel's code
// buffers after its main loop and a barrier) of at least NW * 32 * RS bytes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "codec.hpp"

namespace bsq {
namespace epi {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Staged row stride in bytes (padded against bank conflicts).
template <int WTN, int ES> constexpr int row_stride() { return WTN * ES + 16; }
// LDS bytes the call needs for NW waves (the f32 case is the larger).
template <int WTN, int NW> constexpr int stage_bytes() { return NW * 32 * row_stride<WTN, 4>(); }

template <int MT, int NT, int WTN, int ES>
__device__ __forceinline__ void store_es(const f32x16_t (&acc)[MT][NT], float scale, uint8_t *st, int lane,
                                         int64_t r0, int64_t c0, int64_t m, int64_t n, void *out,
                                         const int32_t *rowmap) {
  constexpr int EV = 16 / ES;                // elements per 16-byte piece
  constexpr int RS = row_stride<WTN, ES>();  // staged row stride
  constexpr int LPR = WTN * ES / 16;         // lanes per staged row
  constexpr int RPI = 64 / LPR;              // rows per read-back instruction
  static_assert(LPR >= 1 && 64 % LPR == 0 && 32 % RPI == 0, "tile width must give whole 16-byte pieces");
  const int l32 = lane & 31, h = lane >> 5;
  const bool vec = n % EV == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  const int lr = lane / LPR, lc = (lane % LPR) * EV;
  const int64_t gc = c0 + lc;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = (v >> 2) * 8 + h * 4 + (v & 3), c = j * 32 + l32;
        const float val = acc[i][j][v] * scale;
        if constexpr (ES == 4) *reinterpret_cast<float *>(st + r * RS + c * 4) = val;
        else *reinterpret_cast<uint16_t *>(st + r * RS + c * 2) = f32_to_bf16_bits(val);
      }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 32 / RPI; ++q) {
      const int r = q * RPI + lr;
      const u32x4_t val = *reinterpret_cast<const u32x4_t *>(st + r * RS + lc * ES);
      const int64_t gr = r0 + i * 32 + r;
      if (gr >= m) continue;
      const int64_t orow = rowmap ? (int64_t)rowmap[gr] : gr;
      uint8_t *dst = reinterpret_cast<uint8_t *>(out) + (orow * n + gc) * ES;
      if (vec && gc + EV <= n) {
        __builtin_nontemporal_store(val, reinterpret_cast<u32x4_t *>(dst));
      } else {
#pragma unroll
        for (int e = 0; e < EV; ++e) {
          const uint32_t word = val[e * ES / 4];
          if (gc + e < n) {
            if constexpr (ES == 4) reinterpret_cast<uint32_t *>(dst)[e] = word;
            else reinterpret_cast<uint16_t *>(dst)[e] = (uint16_t)(word >> (16 * (e & 1)));
          }
        }
      }
    }
    __syncthreads();
  }
}

// acc: this wave's MT x NT tiles; the wave's output block starts at row r0,
// column c0; stage: this wave's own LDS region.  Every wave of the workgroup
// must call it (it synchronizes the workgroup once per band).  ot: 0 = f32,
// 1 = bf16.  Each value is multiplied by scale before rounding.  Rows at or
// past m are not written; rowmap (may be null) sends row r to output row
// rowmap[r] (the expert-grouped GEMM's token rows).
template <int MT, int NT, int WTN>
__device__ __forceinline__ void store_acc(const f32x16_t (&acc)[MT][NT], float scale, uint8_t *stage, int lane,
                                          int64_t r0, int64_t c0, int64_t m, int64_t n, void *out, int ot,
                                          const int32_t *rowmap = nullptr) {
  if (ot == 0) store_es<MT, NT, WTN, 4>(acc, scale, stage, lane, r0, c0, m, n, out, rowmap);
  else store_es<MT, NT, WTN, 2>(acc, scale, stage, lane, r0, c0, m, n, out, rowmap);
}

}  // namespace epi
}  // namespace bsq
