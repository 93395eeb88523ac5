// bsq_internal.hpp -- format traits and kernel launchers shared by the
// library's translation units (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsq {

enum Fmt : int {
  kMXFP4 = 1,
  kNVFP4 = 2,
  kMXFP8_E4M3 = 3,
  kMXFP8_E5M2 = 4,
  kNVFP8 = 5,
  kINT4_AFFINE = 6,
  kINT8_SYM = 7
};

// Compile-time description of each format's storage.
template <int F> struct Traits;
template <> struct Traits<kMXFP4> { static constexpr int kBlock = 32, kBits = 4; };
template <> struct Traits<kNVFP4> { static constexpr int kBlock = 16, kBits = 4; };
template <> struct Traits<kMXFP8_E4M3> { static constexpr int kBlock = 32, kBits = 8; };
template <> struct Traits<kMXFP8_E5M2> { static constexpr int kBlock = 32, kBits = 8; };
template <> struct Traits<kNVFP8> { static constexpr int kBlock = 16, kBits = 8; };
template <> struct Traits<kINT4_AFFINE> { static constexpr int kBlock = 64, kBits = 4; };
template <> struct Traits<kINT8_SYM> { static constexpr int kBlock = 32, kBits = 8; };

inline int block_of(int f) {
  switch (f) {
    case kMXFP4: case kMXFP8_E4M3: case kMXFP8_E5M2: case kINT8_SYM: return 32;
    case kNVFP4: case kNVFP8: return 16;
    case kINT4_AFFINE: return 64;
    default: return 0;
  }
}
inline bool is_4bit(int f) { return f == kMXFP4 || f == kNVFP4 || f == kINT4_AFFINE; }

// A packed weight as the kernels see it (all device pointers).
struct QWeight {
  int fmt;
  int64_t n, k;
  const void *codes, *scales, *biases;
  float global;
};

// Launchers (defined in the .hip files).  Shapes are validated by the caller.
hipError_t launch_dequant(const QWeight &w, float *out, hipStream_t s);
// VALU streaming kernel: any m, f32 or bf16 X (xt/ot: 0 = f32, 1 = bf16).
hipError_t launch_rows(const QWeight &w, int64_t m, const void *x, int xt, void *out, int ot, hipStream_t s);
// The same kernel with the fused RMSNorm of each X row: gamma [k] of dtype xt,
// out = (x * gamma / sqrt(mean(x^2) + eps)) . dequant(W)^T; k % 32 == 0 for
// 4-bit formats.
hipError_t launch_rows_norm(const QWeight &w, int64_t m, const void *x, int xt, const void *gam, float eps, void *out,
                            int ot, hipStream_t s);
// Expert-routed rows: w is one expert's shape (n rows) over a stacked [E*n, k]
// weight; X row i uses expert eids[i] (device int32 [m]); a bad id zeroes the
// row and sets *status (may be null) to 1.
hipError_t launch_rows_gather(const QWeight &w, int64_t m, const void *x, int xt, const int32_t *eids, int64_t nexp,
                              int *status, void *out, int ot, hipStream_t s);
// Decode GEMV kernel (gemv.hip): bf16 activation rows that each stream the
// weight once (m == 1, or every routed row when routed), whole 16-byte code
// chunks (k % 32 == 0 for 4-bit codes, k % 16 == 0 for 8-bit).
bool gemv_applies(const QWeight &w, int64_t m, int xt, bool routed);
hipError_t launch_gemv(const QWeight &w, int64_t m, const void *x, void *out, int ot, const int32_t *eids,
                       int64_t nexp, int *status, hipStream_t s);
// The fused RMSNorm on the decode GEMV kernel: up to kGemvNormRows bf16 rows
// (one grid row each), k = 64 chunks per wave of the k split (4096 for every
// format).
constexpr int64_t kGemvNormRows = 32;
bool gemv_norm_applies(const QWeight &w, int64_t m, int xt);
hipError_t launch_gemv_norm(const QWeight &w, int64_t m, const void *x, const void *gam, float eps, void *out, int ot,
                            hipStream_t s);
// The decode form of the expert-grouped matmul on the decode GEMV kernel
// (gemv.hip): routed in the kernel itself, tiles of up to kGemvGroupRows rows
// of one expert, one pass over the expert's weight per tile; bad ids zero
// their rows and set *status (may be null) to 1.  Applies to m up to
// kGemvGroupMaxRows, whole 16-byte code chunks, and 31-bit offsets of the
// stacked weight and of the m rows.
// With eids null the same kernel runs m dense rows of one weight (nexp 1) in
// tiles of kGemvGroupRows consecutive rows: the small-m bf16 product takes it
// for 2 <= m <= kGemvDenseRows.
constexpr int kGemvGroupRows = 4;
constexpr int64_t kGemvGroupMaxRows = 32;
constexpr int64_t kGemvDenseRows = 32;
bool gemv_grouped_applies(const QWeight &w, int64_t m, int64_t nexp);
// Whether bf16 X of m rows is better served by that multi-row form than by
// the MFMA kernel (measured crossover: m <= 8, or m <= 32 while ceil(m/4)
// passes over the packed weight stay within 96 MB).
bool gemv_dense_preferred(const QWeight &w, int64_t m);
hipError_t launch_gemv_grouped(const QWeight &w, int64_t m, int64_t nexp, const int32_t *eids, const void *x,
                               void *out, int ot, int *status, hipStream_t s);
// MFMA kernel: bf16 X, any m >= 1.
hipError_t launch_mfma(const QWeight &w, int64_t m, const void *x, void *out, int ot, hipStream_t s);
// Zero-fill an output of `bytes` bytes (k == 0 case).
hipError_t launch_zero(void *out, int64_t bytes, hipStream_t s);

// Device packer (quantize.hip): the host packer's encoding on the GPU.  gdev
// (nvfp4) receives the global scale; status (may be null) receives 5 if a
// block holds a non-finite value.
hipError_t launch_quantize(int fmt, const void *w, int wt, int64_t n, int64_t k, void *codes, void *scales,
                           void *biases, float *gdev, int *status, hipStream_t s);
// Scaled-MFMA GEMM (mxmma.hip): both operands MX-packed (mxfp4 / mxfp8),
// k a multiple of 128.
hipError_t launch_mxmma(int xfmt, const void *xc, const void *xs, int wfmt, const void *wc, const void *ws, int64_t m,
                        int64_t n, int64_t k, void *out, int ot, hipStream_t s);

// Expert-grouped GEMM (grouped.hip): bf16 X [m,k], expert ids [m], a stacked
// [E*n, k] weight (w.n = n, the rows of one expert); workspace of
// grouped_workspace_bytes(m, E) bytes holds the routing table.
constexpr int kMaxExperts = 1024;
int64_t grouped_workspace_bytes(int64_t m, int64_t nexp);
// The routing table of the allocation-free grouped call: a file-scope device
// array of this many bytes in grouped.hip; grouped_scratch gives its address
// on the current device (looked up once per device).
constexpr int64_t kNoAllocTableBytes = (int64_t)1 << 20;
constexpr int kMaxDevices = 64;
hipError_t grouped_scratch(void **ptr);
hipError_t launch_grouped(const QWeight &w, int64_t m, int64_t nexp, const int32_t *eids, const void *x, void *out,
                          int ot, void *workspace, int *status, hipStream_t s);
// The grouped form of the MFMA kernel (mfma.hip) over a routing table: gtab[0]
// tiles, (expert, first row, row end) per tile, tokens at gtab + gperm.
hipError_t launch_mfma_grouped(const QWeight &w, int64_t m, const void *x, void *out, int ot, const int32_t *gtab,
                               int64_t gperm, int tiles_m, hipStream_t s);

// Calibration kernels (calib.hip): streaming read of `bytes` (a multiple of
// 16) and a register-only bf16 MFMA loop.
hipError_t launch_calib_read(const void *buf, int64_t bytes, float *sink, hipStream_t s);
hipError_t launch_calib_mfma(int64_t iters, int64_t workgroups, float *sink, hipStream_t s);

// Host packer (pack_host.cpp).  Returns a bsq_status value.
int pack_host(int fmt, const float *w, int64_t n, int64_t k, void *codes, void *scales, void *biases,
              float *global_out);

}  // namespace bsq
