// grouped.hip -- expert-grouped quantized matmul for prefill-scale MoE:
//   out[i,j] = sum_p X[i,p] * dequant(W)[expert_ids[i]*n + j, p]
// over one stacked [E*n, k] packed weight [metaltile PR #250, commit adding
// the per-token expert-routed qmm: the weight row is expert_ids[m]*out_dim +
// n; rlx-cpu quant.rs, lowp_scaled_grouped_matmul: the expert-indexed GEMM].
// The result is the routed gather's, row for row; what differs is the
// schedule: rows are grouped by expert so each expert's weight tile is
// streamed once per 128 routed rows through the bf16 MFMA kernel, instead of
// once per routed row.
//
//  1. route_kernel (one workgroup): counts the rows of each expert in LDS,
//     scans the counts and the 128-row tile counts, and writes the routing
//     table: the number of tiles, each tile's (expert, first sorted row, end of
//     its expert's rows), and the token of every sorted row.  Rows whose id
//     is outside [0, E) are written as zeros and flag *status.
//  2. mfma_kernel in its grouped form (mfma.hip): X rows gathered and output
//     rows scattered through the table; tiles past the count exit at once.
// Decode-sized m (at most 32 rows, 31-bit offsets) skips both: the GEMV
// kernel's grouped form (gemv.hip) routes the few rows itself and streams
// each expert's weight once per tile of up to 4 of its rows.
// The order of rows inside an expert's group comes from LDS atomics, but every
// output row is computed the same way wherever it sits, so the result is
// bit-for-bit the same from run to run.
#include <mutex>

#include "bsq_internal.hpp"

namespace bsq {
namespace {

constexpr int kRouteThreads = 1024;
constexpr int kTileRows = 128;  // rows per m-tile of the grouped GEMM configurations

// Inclusive sum over the workgroup of one int per thread (kRouteThreads
// threads, 16 waves); `tmp` holds 16 wave totals.  Every thread gets its
// inclusive prefix; *total receives the sum.
__device__ __forceinline__ int block_inclusive_scan(int v, int *tmp, int *total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  if (lane == 63) tmp[w] = v;
  __syncthreads();
  if (w == 0) {
    int t = lane < kRouteThreads / 64 ? tmp[lane] : 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int o = __shfl_up(t, d);
      if (lane >= d) t += o;
    }
    if (lane < kRouteThreads / 64) tmp[lane] = t;  // inclusive wave totals
  }
  __syncthreads();
  const int r = v + (w > 0 ? tmp[w - 1] : 0);
  if (threadIdx.x == kRouteThreads - 1) *total = r;
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(kRouteThreads)
route_kernel(const int32_t *__restrict__ eids, int64_t m, int nexp, int32_t *__restrict__ table, int64_t perm_off,
             void *__restrict__ out, int ot, int64_t n, int *__restrict__ status) {
  __shared__ int cnt[kMaxExperts], cur[kMaxExperts];
  __shared__ int tmp[kRouteThreads / 64], tot_rows, tot_tiles;
  const int t = threadIdx.x;
  for (int e = t; e < nexp; e += kRouteThreads) cnt[e] = 0;
  __syncthreads();
  bool bad = false;
  for (int64_t i = t; i < m; i += kRouteThreads) {
    const int e = eids[i];
    if (e >= 0 && e < nexp) {
      atomicAdd(&cnt[e], 1);
    } else {  // an id outside [0, E): the row is zeros
      bad = true;
      if (ot == 0) {
        float *row = reinterpret_cast<float *>(out) + i * n;
        for (int64_t j = 0; j < n; ++j) row[j] = 0.0f;
      } else {
        uint16_t *row = reinterpret_cast<uint16_t *>(out) + i * n;
        for (int64_t j = 0; j < n; ++j) row[j] = 0;
      }
    }
  }
  if (bad && status) *status = 1;
  __syncthreads();
  // thread e owns expert e (nexp <= kRouteThreads): row offset and tile offset
  const int c = t < nexp ? cnt[t] : 0;
  const int tiles = (c + kTileRows - 1) / kTileRows;
  const int row_end = block_inclusive_scan(c, tmp, &tot_rows);
  const int tile_end = block_inclusive_scan(tiles, tmp, &tot_tiles);
  const int row0 = row_end - c, tile0 = tile_end - tiles;
  if (t < nexp) {
    cur[t] = row0;
    for (int q = 0; q < tiles; ++q) {
      int32_t *tile = table + 1 + 3 * (int64_t)(tile0 + q);
      tile[0] = t;                     // expert
      tile[1] = row0 + q * kTileRows;  // first sorted row of the tile
      tile[2] = row_end;               // end of the expert's rows
    }
  }
  if (t == 0) table[0] = tot_tiles;
  __syncthreads();
  int32_t *perm = table + perm_off;
  for (int64_t i = t; i < m; i += kRouteThreads) {
    const int e = eids[i];
    if (e >= 0 && e < nexp) perm[atomicAdd(&cur[e], 1)] = (int32_t)i;
  }
}

// The routing table for m rows and E experts, in int32 words: the tile
// count, (expert, first row, row end) per possible tile, then the tokens.
int64_t max_tiles(int64_t m, int64_t nexp) { return (m + kTileRows - 1) / kTileRows + (nexp < m ? nexp : m); }
int64_t perm_offset(int64_t m, int64_t nexp) { return 1 + 3 * max_tiles(m, nexp); }
int64_t table_words(int64_t m, int64_t nexp) { return perm_offset(m, nexp) + m; }

}  // namespace

// ---- the routing table of the allocation-free call ----
//
// A file-scope device array, one per device the library runs on, held until
// the process ends.  Its host-side name is not a device address: its address
// on each device is looked up once, with that device current, and only that
// address is handed to kernels.  Every allocation-free call on a device
// shares the device's table, so such calls that overlap on one device race.
// Nothing in it needs to start at zero: the route kernel writes every word a
// call then reads (tile count, tile entries, sorted rows) before the GEMM.
static __device__ __align__(256) int32_t scratch[kNoAllocTableBytes / 4];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t grouped_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

int64_t grouped_workspace_bytes(int64_t m, int64_t nexp) { return 4 * table_words(m, nexp); }

hipError_t launch_grouped(const QWeight &w, int64_t m, int64_t nexp, const int32_t *eids, const void *x, void *out,
                          int ot, void *workspace, int *status, hipStream_t s) {
  if (gemv_grouped_applies(w, m, nexp)) return launch_gemv_grouped(w, m, nexp, eids, x, out, ot, status, s);
  int32_t *table = reinterpret_cast<int32_t *>(workspace);
  const int64_t poff = perm_offset(m, nexp);
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), 0, s, eids, m, (int)nexp, table, poff, out, ot,
                     w.n, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_mfma_grouped(w, m, x, out, ot, table, poff, (int)max_tiles(m, nexp), s);
}

}  // namespace bsq
