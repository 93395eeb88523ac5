// lds_swizzle.hpp -- bank-conflict-free placement of row tiles in LDS.
//
// A tile of rows of RB bytes (RB a multiple of 16, at most 256) is stored
// row-major with the 16-byte chunk index of row r XORed with a key of r.  A
// 16-byte LDS access serves 16 lanes per pass over 64 banks x 4 bytes, so it
// is conflict free when those lanes' 16-byte granules fall on 16 distinct
// positions modulo 256 bytes.  The key makes that hold both for 16
// consecutive rows at one chunk (the MFMA operand reads: one row per lane)
// and for the chunks of consecutive rows (a row-major fill).
#pragma once
#include <hip/hip_runtime.h>

namespace bsq {

template <int RB> struct Swz {
  static_assert(RB % 16 == 0 && RB <= 256 && 256 % RB == 0, "rows of 16 to 256 bytes dividing 256");
  static constexpr int kCPR = RB / 16, kRPB = 256 / RB;
  static constexpr int kPeriod = kCPR * kRPB;  // rows after which the key repeats
  __device__ static int key(int r) { return (r / kRPB) % kCPR; }
  // byte offset of 16-byte chunk c of row r
  __device__ static int at(int r, int c) { return r * RB + ((c ^ key(r)) << 4); }
};

}  // namespace bsq
