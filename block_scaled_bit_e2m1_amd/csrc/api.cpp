// api.cpp -- the C ABI: argument validation, kernel-family dispatch, errors.
//
// Every check happens before any launch; a failing call launches nothing and
// leaves a one-line reason in a thread-local buffer (bsq_last_error).  The
// pages' CPU code panics on an unsupported scheme or a bad shape [rlx-cpu
// quant.rs, compile_dequant_mat_mul and validate_dequant_matmul_dims]; a C ABI
// cannot unwind, so those become status codes here.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/bsq.h"
#include "bsq_internal.hpp"

namespace {

thread_local char g_err[512] = "";

bsq_status fail(bsq_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

bsq_status ok() {
  g_err[0] = 0;
  return BSQ_OK;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bsq_status check_format(int fmt, int block) {
  const int B = bsq::block_of(fmt);
  if (!B) return fail(BSQ_ERR_UNSUPPORTED, "unknown format %d", fmt);
  if (block != 0 && block != B)
    return fail(BSQ_ERR_UNSUPPORTED, "format %d has block %d, got %d", fmt, B, block);
  return BSQ_OK;
}

bsq_status check_shape(int fmt, int64_t n, int64_t k) {
  if (n < 0 || k < 0) return fail(BSQ_ERR_ARG, "negative size n=%lld k=%lld", (long long)n, (long long)k);
  const int B = bsq::block_of(fmt);
  if (k % B) return fail(BSQ_ERR_SHAPE, "k=%lld is not a multiple of the block %d", (long long)k, B);
  if (n > ((int64_t)1 << 40) / (k ? k : 1)) return fail(BSQ_ERR_SHAPE, "n*k too large");
  return BSQ_OK;
}

size_t scale_elem_bytes(int fmt) {
  switch (fmt) {
    case bsq::kNVFP8: case bsq::kINT8_SYM: return 4;
    case bsq::kINT4_AFFINE: return 2;
    default: return 1;
  }
}

bsq_status check_weight(int fmt, int64_t n, int64_t k, const void *codes, const void *scales, const void *biases) {
  if (n == 0 || k == 0) return BSQ_OK;
  if (!codes || !scales) return fail(BSQ_ERR_ARG, "null codes or scales");
  if (fmt == bsq::kINT4_AFFINE && !biases) return fail(BSQ_ERR_ARG, "int4 affine needs biases");
  if (!aligned(codes, 16)) return fail(BSQ_ERR_ALIGN, "codes must be 16-byte aligned");
  if (!aligned(scales, scale_elem_bytes(fmt))) return fail(BSQ_ERR_ALIGN, "scales misaligned");
  if (biases && !aligned(biases, 2)) return fail(BSQ_ERR_ALIGN, "biases misaligned");
  return BSQ_OK;
}

bsq_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(BSQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bsq_status matmul(bsq_path path, bsq_format fmt, int block, int64_t m, int64_t n, int64_t k, const void *codes,
                  const void *scales, const void *biases, float global_scale, const void *x, bsq_dtype xt,
                  void *out, bsq_dtype ot, void *stream) {
  bsq_status s;
  if ((s = check_format(fmt, block))) return s;
  if ((s = check_shape(fmt, n, k))) return s;
  if (m < 0) return fail(BSQ_ERR_ARG, "negative m");
  if (xt != BSQ_F32 && xt != BSQ_BF16) return fail(BSQ_ERR_ARG, "bad x dtype %d", (int)xt);
  if (ot != BSQ_F32 && ot != BSQ_BF16) return fail(BSQ_ERR_ARG, "bad out dtype %d", (int)ot);
  if (path != BSQ_PATH_AUTO && path != BSQ_PATH_ROWS && path != BSQ_PATH_MFMA)
    return fail(BSQ_ERR_ARG, "bad path %d", (int)path);
  if (path == BSQ_PATH_MFMA && xt != BSQ_BF16)
    return fail(BSQ_ERR_UNSUPPORTED, "the MFMA path takes bf16 X");
  if (m == 0 || n == 0) return ok();
  if (!out) return fail(BSQ_ERR_ARG, "null out");
  if (!aligned(out, ot == BSQ_F32 ? 4 : 2)) return fail(BSQ_ERR_ALIGN, "out misaligned");
  hipStream_t st = (hipStream_t)stream;
  const int64_t ob = m * n * (ot == BSQ_F32 ? 4 : 2);
  if (k == 0) return hip_status(bsq::launch_zero(out, ob, st), "zero-fill");
  if ((s = check_weight(fmt, n, k, codes, scales, biases))) return s;
  if (!x) return fail(BSQ_ERR_ARG, "null x");
  if (!aligned(x, 16)) return fail(BSQ_ERR_ALIGN, "x must be 16-byte aligned");
  if (m > ((int64_t)1 << 40) / k) return fail(BSQ_ERR_SHAPE, "m*k too large");
  const bsq::QWeight w{(int)fmt, n, k, codes, scales, biases, global_scale};
  if (path == BSQ_PATH_AUTO)
    path = (xt == BSQ_BF16 && m > 8 && !bsq::gemv_dense_preferred(w, m)) ? BSQ_PATH_MFMA : BSQ_PATH_ROWS;
  if (path == BSQ_PATH_MFMA) return hip_status(bsq::launch_mfma(w, m, x, out, (int)ot, st), "mfma launch");
  return hip_status(bsq::launch_rows(w, m, x, (int)xt, out, (int)ot, st), "rows launch");
}

}  // namespace

extern "C" {

bsq_status bsq_packed_bytes(bsq_format fmt, int block, int64_t n, int64_t k, size_t *code_bytes,
                            size_t *scale_bytes, size_t *bias_bytes) {
  bsq_status s;
  if ((s = check_format(fmt, block))) return s;
  if ((s = check_shape(fmt, n, k))) return s;
  const int64_t nb = n * (k / bsq::block_of(fmt));
  if (code_bytes) *code_bytes = (size_t)(bsq::is_4bit(fmt) ? n * k / 2 : n * k);
  if (scale_bytes) *scale_bytes = (size_t)nb * scale_elem_bytes(fmt);
  if (bias_bytes) *bias_bytes = fmt == BSQ_INT4_AFFINE ? (size_t)nb * 2 : 0;
  return ok();
}

bsq_status bsq_pack_host(bsq_format fmt, int block, const float *w, int64_t n, int64_t k, void *codes,
                         void *scales, void *biases, float *global_out) {
  bsq_status s;
  if ((s = check_format(fmt, block))) return s;
  if ((s = check_shape(fmt, n, k))) return s;
  if (n * k > 0 && (!w || !codes || !scales)) return fail(BSQ_ERR_ARG, "null pointer");
  if (n * k > 0 && fmt == BSQ_INT4_AFFINE && !biases) return fail(BSQ_ERR_ARG, "int4 affine needs biases");
  const int st = bsq::pack_host(fmt, w, n, k, codes, scales, biases, global_out);
  if (st) return fail((bsq_status)st, "non-finite weight value");
  return ok();
}

bsq_status bsq_quantize(bsq_format fmt, int block, const void *w, bsq_dtype wt, int64_t n, int64_t k, void *codes,
                        void *scales, void *biases, float *global_dev, int *status_dev, void *stream) {
  bsq_status s;
  if ((s = check_format(fmt, block))) return s;
  if ((s = check_shape(fmt, n, k))) return s;
  if (wt != BSQ_F32 && wt != BSQ_BF16) return fail(BSQ_ERR_ARG, "bad input dtype %d", (int)wt);
  if (n == 0 || k == 0) return ok();
  if (!w || !codes || !scales) return fail(BSQ_ERR_ARG, "null pointer");
  if (fmt == BSQ_INT4_AFFINE && !biases) return fail(BSQ_ERR_ARG, "int4 affine needs biases");
  if (fmt == BSQ_NVFP4 && !global_dev) return fail(BSQ_ERR_ARG, "nvfp4 needs a device float for the global scale");
  if (!aligned(w, 16) || !aligned(codes, 16)) return fail(BSQ_ERR_ALIGN, "w and codes must be 16-byte aligned");
  if (!aligned(scales, scale_elem_bytes(fmt)) || (biases && !aligned(biases, 2)) ||
      (global_dev && !aligned(global_dev, 4)) || (status_dev && !aligned(status_dev, 4)))
    return fail(BSQ_ERR_ALIGN, "scales, biases, global or status misaligned");
  return hip_status(bsq::launch_quantize(fmt, w, (int)wt, n, k, codes, scales, biases, global_dev, status_dev,
                                         (hipStream_t)stream),
                    "quantize launch");
}

bsq_status bsq_qgemm_mx(bsq_format xfmt, const void *x_codes, const void *x_scales, bsq_format wfmt,
                        const void *w_codes, const void *w_scales, int64_t m, int64_t n, int64_t k, void *out,
                        bsq_dtype ot, void *stream) {
  auto is_mx = [](int f) { return f == BSQ_MXFP4 || f == BSQ_MXFP8_E4M3 || f == BSQ_MXFP8_E5M2; };
  if (!is_mx(xfmt) || !is_mx(wfmt)) return fail(BSQ_ERR_UNSUPPORTED, "both operands must be MX formats");
  if (m < 0 || n < 0 || k < 0) return fail(BSQ_ERR_ARG, "negative size");
  if (k % 128) return fail(BSQ_ERR_SHAPE, "k=%lld is not a multiple of 128", (long long)k);
  if (ot != BSQ_F32 && ot != BSQ_BF16) return fail(BSQ_ERR_ARG, "bad out dtype %d", (int)ot);
  if (m == 0 || n == 0) return ok();
  if (!out) return fail(BSQ_ERR_ARG, "null out");
  if (!aligned(out, ot == BSQ_F32 ? 4 : 2)) return fail(BSQ_ERR_ALIGN, "out misaligned");
  hipStream_t st = (hipStream_t)stream;
  if (k == 0) return hip_status(bsq::launch_zero(out, m * n * (ot == BSQ_F32 ? 4 : 2), st), "zero-fill");
  if (m > ((int64_t)1 << 40) / k || n > ((int64_t)1 << 40) / k) return fail(BSQ_ERR_SHAPE, "sizes too large");
  if (!x_codes || !x_scales || !w_codes || !w_scales) return fail(BSQ_ERR_ARG, "null pointer");
  if (!aligned(x_codes, 16) || !aligned(w_codes, 16)) return fail(BSQ_ERR_ALIGN, "codes must be 16-byte aligned");
  if (!aligned(x_scales, 4) || !aligned(w_scales, 4)) return fail(BSQ_ERR_ALIGN, "scales must be 4-byte aligned");
  return hip_status(bsq::launch_mxmma(xfmt, x_codes, x_scales, wfmt, w_codes, w_scales, m, n, k, out, (int)ot, st),
                    "mx mfma launch");
}

bsq_status bsq_dequant(bsq_format fmt, int block, int64_t n, int64_t k, const void *codes, const void *scales,
                       const void *biases, float global_scale, float *out, void *stream) {
  bsq_status s;
  if ((s = check_format(fmt, block))) return s;
  if ((s = check_shape(fmt, n, k))) return s;
  if (n == 0 || k == 0) return ok();
  if ((s = check_weight(fmt, n, k, codes, scales, biases))) return s;
  if (!out) return fail(BSQ_ERR_ARG, "null out");
  if (!aligned(out, 16)) return fail(BSQ_ERR_ALIGN, "out must be 16-byte aligned");
  const bsq::QWeight w{(int)fmt, n, k, codes, scales, biases, global_scale};
  return hip_status(bsq::launch_dequant(w, out, (hipStream_t)stream), "dequant launch");
}

bsq_status bsq_qgemv(bsq_format fmt, int block, int64_t n, int64_t k, const void *codes, const void *scales,
                     const void *biases, float global_scale, const void *x, bsq_dtype xt, void *out,
                     bsq_dtype ot, void *stream) {
  return matmul(BSQ_PATH_ROWS, fmt, block, 1, n, k, codes, scales, biases, global_scale, x, xt, out, ot, stream);
}

bsq_status bsq_qgemm(bsq_format fmt, int block, int64_t m, int64_t n, int64_t k, const void *codes,
                     const void *scales, const void *biases, float global_scale, const void *x, bsq_dtype xt,
                     void *out, bsq_dtype ot, void *stream) {
  return matmul(BSQ_PATH_AUTO, fmt, block, m, n, k, codes, scales, biases, global_scale, x, xt, out, ot, stream);
}

bsq_status bsq_qgemm_path(bsq_path path, bsq_format fmt, int block, int64_t m, int64_t n, int64_t k,
                          const void *codes, const void *scales, const void *biases, float global_scale,
                          const void *x, bsq_dtype xt, void *out, bsq_dtype ot, void *stream) {
  return matmul(path, fmt, block, m, n, k, codes, scales, biases, global_scale, x, xt, out, ot, stream);
}

bsq_status bsq_rmsnorm_qgemv(bsq_format fmt, int block, int64_t m, int64_t n, int64_t k, const void *codes,
                             const void *scales, const void *biases, float global_scale, const void *x,
                             const void *norm_weight, float eps, bsq_dtype xt, void *out, bsq_dtype ot,
                             void *stream) {
  bsq_status s;
  if ((s = check_format(fmt, block))) return s;
  if ((s = check_shape(fmt, n, k))) return s;
  if (m < 0) return fail(BSQ_ERR_ARG, "negative m");
  if (xt != BSQ_F32 && xt != BSQ_BF16) return fail(BSQ_ERR_ARG, "bad x dtype %d", (int)xt);
  if (ot != BSQ_F32 && ot != BSQ_BF16) return fail(BSQ_ERR_ARG, "bad out dtype %d", (int)ot);
  if (!(eps >= 0.0f) || eps > 3.0e38f) return fail(BSQ_ERR_ARG, "eps must be finite and >= 0");
  if (bsq::is_4bit(fmt) && k % 32) return fail(BSQ_ERR_SHAPE, "k=%lld: 4-bit formats need k %% 32 == 0 here", (long long)k);
  if (m == 0 || n == 0) return ok();
  if (!out) return fail(BSQ_ERR_ARG, "null out");
  if (!aligned(out, ot == BSQ_F32 ? 4 : 2)) return fail(BSQ_ERR_ALIGN, "out misaligned");
  hipStream_t st = (hipStream_t)stream;
  if (k == 0) return hip_status(bsq::launch_zero(out, m * n * (ot == BSQ_F32 ? 4 : 2), st), "zero-fill");
  if ((s = check_weight(fmt, n, k, codes, scales, biases))) return s;
  if (!x || !norm_weight) return fail(BSQ_ERR_ARG, "null x or norm_weight");
  if (!aligned(x, 16) || !aligned(norm_weight, 16)) return fail(BSQ_ERR_ALIGN, "x and norm_weight must be 16-byte aligned");
  if (m > ((int64_t)1 << 40) / k) return fail(BSQ_ERR_SHAPE, "m*k too large");
  const bsq::QWeight w{(int)fmt, n, k, codes, scales, biases, global_scale};
  if (bsq::gemv_norm_applies(w, m, (int)xt))
    return hip_status(bsq::launch_gemv_norm(w, m, x, norm_weight, eps, out, (int)ot, st), "rmsnorm gemv launch");
  return hip_status(bsq::launch_rows_norm(w, m, x, (int)xt, norm_weight, eps, out, (int)ot, st), "rmsnorm rows launch");
}

bsq_status bsq_gather_qmm(bsq_format fmt, int block, int64_t m, int64_t n, int64_t k, int64_t num_experts,
                          const void *codes, const void *scales, const void *biases, float global_scale,
                          const int32_t *expert_ids, const void *x, bsq_dtype xt, void *out, bsq_dtype ot,
                          int *status_dev, void *stream) {
  bsq_status s;
  if ((s = check_format(fmt, block))) return s;
  if (num_experts < 1) return fail(BSQ_ERR_ARG, "num_experts must be >= 1");
  if (n < 0 || n > ((int64_t)1 << 40) / num_experts) return fail(BSQ_ERR_SHAPE, "n * num_experts out of range");
  if ((s = check_shape(fmt, n * num_experts, k))) return s;
  if (m < 0) return fail(BSQ_ERR_ARG, "negative m");
  if (m > 65535) return fail(BSQ_ERR_SHAPE, "m=%lld: at most 65535 routed rows per call", (long long)m);
  if (xt != BSQ_F32 && xt != BSQ_BF16) return fail(BSQ_ERR_ARG, "bad x dtype %d", (int)xt);
  if (ot != BSQ_F32 && ot != BSQ_BF16) return fail(BSQ_ERR_ARG, "bad out dtype %d", (int)ot);
  if (m == 0 || n == 0) return ok();
  if (!out) return fail(BSQ_ERR_ARG, "null out");
  if (!aligned(out, ot == BSQ_F32 ? 4 : 2)) return fail(BSQ_ERR_ALIGN, "out misaligned");
  hipStream_t st = (hipStream_t)stream;
  if (k == 0) return hip_status(bsq::launch_zero(out, m * n * (ot == BSQ_F32 ? 4 : 2), st), "zero-fill");
  if ((s = check_weight(fmt, n * num_experts, k, codes, scales, biases))) return s;
  if (!x || !expert_ids) return fail(BSQ_ERR_ARG, "null x or expert_ids");
  if (!aligned(x, 16) || !aligned(expert_ids, 4)) return fail(BSQ_ERR_ALIGN, "x (16) or expert_ids (4) misaligned");
  if (status_dev && !aligned(status_dev, 4)) return fail(BSQ_ERR_ALIGN, "status misaligned");
  const bsq::QWeight w{(int)fmt, n, k, codes, scales, biases, global_scale};
  return hip_status(bsq::launch_rows_gather(w, m, x, (int)xt, expert_ids, num_experts, status_dev, out, (int)ot, st),
                    "gather launch");
}

bsq_status bsq_grouped_qgemm_workspace(int64_t m, int64_t num_experts, size_t *bytes) {
  if (m < 0 || num_experts < 1 || !bytes) return fail(BSQ_ERR_ARG, "bad m, num_experts or null bytes");
  if (num_experts > bsq::kMaxExperts || m > ((int64_t)1 << 24))
    return fail(BSQ_ERR_SHAPE, "num_experts <= %d and m <= 2^24", bsq::kMaxExperts);
  *bytes = (size_t)bsq::grouped_workspace_bytes(m, num_experts);
  return ok();
}

namespace {

// The grouped call's checks and launch; workspace == nullptr && noalloc takes
// the routing table from the library's own device array instead.
bsq_status grouped(bsq_format fmt, int block, int64_t m, int64_t n, int64_t k, int64_t num_experts, const void *codes,
                   const void *scales, const void *biases, float global_scale, const int32_t *expert_ids,
                   const void *x, void *out, bsq_dtype ot, void *workspace, size_t workspace_bytes, bool noalloc,
                   int *status_dev, void *stream) {
  bsq_status s;
  if ((s = check_format(fmt, block))) return s;
  if (num_experts < 1) return fail(BSQ_ERR_ARG, "num_experts must be >= 1");
  if (num_experts > bsq::kMaxExperts) return fail(BSQ_ERR_SHAPE, "at most %d experts", bsq::kMaxExperts);
  if (n < 0 || n > ((int64_t)1 << 40) / num_experts) return fail(BSQ_ERR_SHAPE, "n * num_experts out of range");
  if ((s = check_shape(fmt, n * num_experts, k))) return s;
  if (m < 0) return fail(BSQ_ERR_ARG, "negative m");
  if (m > ((int64_t)1 << 24)) return fail(BSQ_ERR_SHAPE, "m=%lld: at most 2^24 rows", (long long)m);
  if (ot != BSQ_F32 && ot != BSQ_BF16) return fail(BSQ_ERR_ARG, "bad out dtype %d", (int)ot);
  if (bsq::is_4bit(fmt) && k % 32) return fail(BSQ_ERR_SHAPE, "k=%lld: 4-bit formats need k %% 32 == 0 here", (long long)k);
  const int64_t need = bsq::grouped_workspace_bytes(m, num_experts);
  if (noalloc && need > bsq::kNoAllocTableBytes)
    return fail(BSQ_ERR_SHAPE, "m=%lld, %lld experts: the routing table needs %lld bytes, the built-in one holds %lld",
                (long long)m, (long long)num_experts, (long long)need, (long long)bsq::kNoAllocTableBytes);
  if (m == 0 || n == 0) return ok();
  if (!out) return fail(BSQ_ERR_ARG, "null out");
  if (!aligned(out, ot == BSQ_F32 ? 4 : 2)) return fail(BSQ_ERR_ALIGN, "out misaligned");
  hipStream_t st = (hipStream_t)stream;
  if (k == 0) return hip_status(bsq::launch_zero(out, m * n * (ot == BSQ_F32 ? 4 : 2), st), "zero-fill");
  if ((s = check_weight(fmt, n * num_experts, k, codes, scales, biases))) return s;
  if (!x || !expert_ids) return fail(BSQ_ERR_ARG, "null x or expert_ids");
  if (!aligned(x, 16) || !aligned(expert_ids, 4)) return fail(BSQ_ERR_ALIGN, "x (16) or expert_ids (4) misaligned");
  if (status_dev && !aligned(status_dev, 4)) return fail(BSQ_ERR_ALIGN, "status misaligned");
  if (m > ((int64_t)1 << 40) / k) return fail(BSQ_ERR_SHAPE, "m*k too large");
  if (noalloc) {
    hipError_t e = bsq::grouped_scratch(&workspace);
    if (e != hipSuccess) return hip_status(e, "routing table lookup");
  } else {
    if (!workspace || (int64_t)workspace_bytes < need)
      return fail(BSQ_ERR_ARG, "workspace of %lld bytes needed", (long long)need);
    if (!aligned(workspace, 4)) return fail(BSQ_ERR_ALIGN, "workspace must be 4-byte aligned");
  }
  const bsq::QWeight w{(int)fmt, n, k, codes, scales, biases, global_scale};
  return hip_status(bsq::launch_grouped(w, m, num_experts, expert_ids, x, out, (int)ot, workspace, status_dev, st),
                    "grouped launch");
}

}  // namespace

bsq_status bsq_grouped_qgemm(bsq_format fmt, int block, int64_t m, int64_t n, int64_t k, int64_t num_experts,
                             const void *codes, const void *scales, const void *biases, float global_scale,
                             const int32_t *expert_ids, const void *x, void *out, bsq_dtype ot, void *workspace,
                             size_t workspace_bytes, int *status_dev, void *stream) {
  return grouped(fmt, block, m, n, k, num_experts, codes, scales, biases, global_scale, expert_ids, x, out, ot,
                 workspace, workspace_bytes, false, status_dev, stream);
}

bsq_status bsq_grouped_qgemm_noalloc(bsq_format fmt, int block, int64_t m, int64_t n, int64_t k, int64_t num_experts,
                                     const void *codes, const void *scales, const void *biases, float global_scale,
                                     const int32_t *expert_ids, const void *x, void *out, bsq_dtype ot,
                                     int *status_dev, void *stream) {
  return grouped(fmt, block, m, n, k, num_experts, codes, scales, biases, global_scale, expert_ids, x, out, ot,
                 nullptr, 0, true, status_dev, stream);
}

bsq_status bsq_calib_read(const void *buf, int64_t bytes, float *sink, void *stream) {
  if (bytes < 0) return fail(BSQ_ERR_ARG, "negative size");
  if (bytes % 16) return fail(BSQ_ERR_SHAPE, "bytes=%lld is not a multiple of 16", (long long)bytes);
  if (bytes == 0) return ok();
  if (!buf || !sink) return fail(BSQ_ERR_ARG, "null buffer or sink");
  if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(BSQ_ERR_ALIGN, "buf must be 16-byte aligned");
  return hip_status(bsq::launch_calib_read(buf, bytes, sink, (hipStream_t)stream), "calib read launch");
}

bsq_status bsq_calib_mfma(int64_t iters, int64_t workgroups, float *sink, void *stream) {
  if (iters < 0 || workgroups < 1 || workgroups > 0x7FFFFFFF) return fail(BSQ_ERR_ARG, "bad iters or workgroups");
  if (!sink || !aligned(sink, 4)) return fail(BSQ_ERR_ARG, "null or misaligned sink");
  return hip_status(bsq::launch_calib_mfma(iters, workgroups, sink, (hipStream_t)stream), "calib mfma launch");
}

const char *bsq_status_string(bsq_status s) {
  switch (s) {
    case BSQ_OK: return "ok";
    case BSQ_ERR_ARG: return "invalid argument";
    case BSQ_ERR_UNSUPPORTED: return "unsupported format or block";
    case BSQ_ERR_SHAPE: return "unsupported shape";
    case BSQ_ERR_ALIGN: return "misaligned pointer";
    case BSQ_ERR_NONFINITE: return "non-finite input";
    case BSQ_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char *bsq_last_error(void) { return g_err; }

const char *bsq_version(void) { return "bsq 0.1.0 (gfx950)"; }

}  // extern "C"
