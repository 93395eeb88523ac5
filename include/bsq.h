/*
 * bsq.h -- block-scaled quantized matmul for AMD Instinct MI355X (gfx950).
 *
 * out[i,j] = sum_p X[i,p] * dequant(W)[j,p]
 *
 * where W is stored as packed low-bit element codes plus one scale per block
 * of consecutive elements along k.  Plain C ABI: every entry point returns a
 * bsq_status, none aborts, throws or allocates caller-visible memory.
 *
 * Formats (element x block x scale), as the pages define them
 * [metaltile PR #250, "complete op x quant-format matrix", table of spec float
 *  formats and commits "Foundation for the spec-conformant ... formats" and
 *  "QFormat {Nvfp4, Mxfp4, Mxfp8E4, Mxfp8E5, Nvfp8} with pack() and dequant()";
 *  metaltile-std tests/qmm_gpu_correctness.rs, int4 affine reference]:
 *
 *   BSQ_MXFP4       E2M1, block 32, E8M0 scale 2^(b-127)
 *   BSQ_NVFP4       E2M1, block 16, E4M3 micro-scale x one f32 global
 *   BSQ_MXFP8_E4M3  E4M3, block 32, E8M0
 *   BSQ_MXFP8_E5M2  E5M2, block 32, E8M0
 *   BSQ_NVFP8       E4M3, block 16, f32 scale
 *   BSQ_INT4_AFFINE unsigned 4-bit q, group 64, value s*q + b (bf16 s and b)
 *   BSQ_INT8_SYM    signed 8-bit q in [-127,127], block 32, f32 scale
 *
 * Stored layouts (all row-major, k contiguous; element (j,p) of W):
 *   4-bit codes: u32 words [n, k/8]; element p sits in word p/8 at bits
 *                4*(p%8)..4*(p%8)+3 (LSB first, low nibble = even element)
 *                [metaltile-std src/mlx/fp_quantized_mma.rs, "W coop-dequant";
 *                 rlx-cpu quant.rs, dequant_matmul_int4 nibble order].
 *   8-bit codes: one byte per element, [n, k].
 *   scales:      [n, k/block]: u8 (E8M0, E4M3), f32 (nvfp8, int8), bf16 bits
 *                as u16 (int4).  int4 biases: bf16 [n, k/64].
 *   X: [m, k] f32 or bf16.  out: [m, n] f32 or bf16 (round to nearest even).
 *
 * Shapes: k must be a multiple of the format's block (BSQ_ERR_SHAPE otherwise);
 * m, n, k may be 0 (nothing is launched; for k == 0 the output is zero-filled).
 * Pointers: device pointers (hipMalloc / torch CUDA tensors) unless marked
 * host.  Codes and X must be 16-byte aligned, out and scales aligned to their
 * element size (BSQ_ERR_ALIGN otherwise).  The caller owns every buffer; the
 * library keeps no state between calls other than the thread-local error text.
 * Device work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 * the default stream); errors detected before launch are returned
 * synchronously, launch failures as BSQ_ERR_HIP.
 */
#ifndef BSQ_H
#define BSQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerated arguments and results are plain ints (the enumerators name
 * the accepted values): a value outside a list reaches the library as an
 * ordinary int and is rejected with a status, never read as an invalid enum. */
enum {
    BSQ_OK = 0,
    BSQ_ERR_ARG = 1,         /* null pointer, negative size, bad dtype */
    BSQ_ERR_UNSUPPORTED = 2, /* unknown format, or block != the format's block */
    BSQ_ERR_SHAPE = 3,       /* k not a multiple of the block, or sizes overflow */
    BSQ_ERR_ALIGN = 4,       /* pointer misaligned for the kernel's vector loads */
    BSQ_ERR_NONFINITE = 5,   /* pack input holds NaN or inf */
    BSQ_ERR_HIP = 6          /* HIP launch / runtime error (see bsq_last_error) */
};
typedef int bsq_status;

enum {
    BSQ_MXFP4 = 1,
    BSQ_NVFP4 = 2,
    BSQ_MXFP8_E4M3 = 3,
    BSQ_MXFP8_E5M2 = 4,
    BSQ_NVFP8 = 5,
    BSQ_INT4_AFFINE = 6,
    BSQ_INT8_SYM = 7
};
typedef int bsq_format;

enum { BSQ_F32 = 0, BSQ_BF16 = 1 };
typedef int bsq_dtype;

/* Kernel family selector for bsq_qgemm_path. */
enum {
    BSQ_PATH_AUTO = 0,  /* library choice by shape and dtype */
    BSQ_PATH_ROWS = 1,  /* VALU streaming kernels: W decoded in registers, dotted with the X rows */
    BSQ_PATH_MFMA = 2   /* LDS-tiled bf16 MFMA kernel (bf16 X only) */
};
typedef int bsq_path;

/* Byte sizes of the packed representation of an [n,k] weight
 * ("byte-layout sizes" [metaltile PR #250, format tests]).  `block` is 0 for
 * the format's block or must equal it.  Any output pointer may be NULL. */
bsq_status bsq_packed_bytes(bsq_format fmt, int block, int64_t n, int64_t k, size_t *code_bytes,
                            size_t *scale_bytes, size_t *bias_bytes);

/* Host packer: f32 weights (host [n,k]) -> codes + scales (+ int4 biases,
 * + nvfp4 global), all host buffers sized by bsq_packed_bytes.
 * Per block along k: the scale is chosen from the block amax (OCP shared
 * exponent for E8M0; nvfp4 two-level global f32(T/2688) with E4M3 micro-scale
 * amax_b/(6g); f32 amax/448 for nvfp8 and amax/127 for int8; bf16 min/max for
 * int4), then every element is encoded against the scale as stored
 * ("pack quantizes against the effective (post-encode) scale"), nearest with
 * ties to even, saturating at the element's largest finite value
 * [metaltile PR #250, QFormat pack commit; rlx-cpu quant.rs,
 *  lowp_compute_scales / lowp_quantize].  `biases` is required for int4 only;
 * `global_out` (may be NULL) receives the nvfp4 global (1.0 otherwise).
 * Returns BSQ_ERR_NONFINITE if w holds NaN or inf (outputs then undefined). */
bsq_status bsq_pack_host(bsq_format fmt, int block, const float *w, int64_t n, int64_t k, void *codes,
                         void *scales, void *biases, float *global_out);

/* Device packer: the same encoding as bsq_pack_host (byte-identical output
 * for f32 input), computed on the GPU from a tensor already in HBM -- the
 * quantize producer of the pages' scaled-matmul ops [rlx-cpu quant.rs,
 * lowp_compute_scales / lowp_quantize; metaltile PR #250, QFormat pack
 * commit].  Used for weights and, with an MX format, for activations.
 * w: device [n,k] of dtype wt (f32, or bf16 whose values are converted to f32
 * exactly), 16-byte aligned.  codes/scales/biases: device buffers
 * sized by bsq_packed_bytes (biases for int4 only).  global_dev: device float,
 * required for nvfp4 (receives f32(T/2688) computed from the tensor amax T on
 * the device; the caller reads it back if it needs it on the host), ignored
 * otherwise.  status_dev: optional device int that the kernel sets to
 * BSQ_ERR_NONFINITE if any weight is NaN or inf (that block's bytes are then
 * unspecified); the caller initialises it.  Asynchronous on `stream`. */
bsq_status bsq_quantize(bsq_format fmt, int block, const void *w, bsq_dtype wt, int64_t n, int64_t k, void *codes,
                        void *scales, void *biases, float *global_dev, int *status_dev, void *stream);

/* Both-operands block-scaled GEMM on the scaled matrix cores:
 *   out[i,j] = sum_p dequant(Xq)[i,p] * dequant(W)[j,p]
 * where Xq (activations, [m,k]) and W ([n,k]) are both packed in an MX format
 * (BSQ_MXFP4, BSQ_MXFP8_E4M3 or BSQ_MXFP8_E5M2: E8M0 scale per 32 along k,
 * stored layouts as above); per block acc += (a_scale * b_scale) *
 * sum dec(a) * dec(b) in fp32 [rlx-cpu quant.rs, lowp_scaled_matmul].  This is
 * an activation-quantized contract: X is first packed with bsq_quantize.
 * k must be a multiple of 128 (BSQ_ERR_SHAPE otherwise); codes 16-byte
 * aligned, scales 4-byte aligned.  out: device [m,n], f32 or bf16 (RNE). */
bsq_status bsq_qgemm_mx(bsq_format xfmt, const void *x_codes, const void *x_scales, bsq_format wfmt,
                        const void *w_codes, const void *w_scales, int64_t m, int64_t n, int64_t k, void *out,
                        bsq_dtype ot, void *stream);

/* Standalone dequant: out (device f32 [n,k]) = decode(code) * scale with one
 * rounding to f32 (nvfp4: (e2m1 * e4m3) * global; int4: s*q + b)
 * [metaltile PR #250, "First spec-conformant block-scaled dequant kernel" and
 *  the commit completing the standalone dequant kernels].  Bit-exact against
 * the CPU definition, NaN and -0 included.  out must be 16-byte aligned. */
bsq_status bsq_dequant(bsq_format fmt, int block, int64_t n, int64_t k, const void *codes,
                       const void *scales, const void *biases, float global_scale, float *out,
                       void *stream);

/* Decode GEMV (m = 1): out[j] = sum_p x[p] * dequant(W)[j,p], fp32
 * accumulation, per-block scale folded once per block and the nvfp4 global
 * once at the end [metaltile PR #250, "First block-scaled matmul kernel:
 * mt_mxfp4_qgemv"; rlx-cpu quant.rs, dequant_matmul_nvfp4].
 * x: device [k] (xt), out: device [n] (ot). */
bsq_status bsq_qgemv(bsq_format fmt, int block, int64_t n, int64_t k, const void *codes, const void *scales,
                     const void *biases, float global_scale, const void *x, bsq_dtype xt, void *out,
                     bsq_dtype ot, void *stream);

/* Multi-row quantized matmul: out[i,j] = sum_p X[i,p] * dequant(W)[j,p]
 * [metaltile PR #250, qmm commit and "mt_mxfp4_qmm_mma" (the M >= 32 path);
 *  metaltile-std src/mlx/fp_quantized_mma.rs, mt_fp4_qmm_mma].  f32 X uses
 * the streaming kernel; bf16 X with m <= 8, or m <= 32 where ceil(m/4) passes
 * over the packed weight stay within 96 MB, the decode GEMV kernel's
 * multi-row form (one weight pass per 4 rows); larger bf16 m the MFMA
 * kernel. */
bsq_status bsq_qgemm(bsq_format fmt, int block, int64_t m, int64_t n, int64_t k, const void *codes,
                     const void *scales, const void *biases, float global_scale, const void *x, bsq_dtype xt,
                     void *out, bsq_dtype ot, void *stream);

/* bsq_qgemm with an explicit kernel family (for cross-path checks: the m = 1
 * result of either family must agree with bsq_qgemv [metaltile-std
 * tests/qmm_gpu_correctness.rs, m=1 qmm vs qmv test]).  BSQ_PATH_MFMA with f32
 * X returns BSQ_ERR_UNSUPPORTED. */
bsq_status bsq_qgemm_path(bsq_path path, bsq_format fmt, int block, int64_t m, int64_t n, int64_t k,
                          const void *codes, const void *scales, const void *biases, float global_scale,
                          const void *x, bsq_dtype xt, void *out, bsq_dtype ot, void *stream);

/* Fused RMSNorm + GEMV: out[i,j] = r_i * sum_p x[i,p] * g[p] * dequant(W)[j,p],
 * r_i = 1 / sqrt(mean_p x[i,p]^2 + eps) [metaltile PR #250, commit adding the
 * block-scaled fused RMSNorm + dequantizing GEMV: phase 1 sums x^2 into the
 * row's inverse RMS, phase 2 is the GEMV over x * norm_weight * inv_rms; the
 * mean over k with eps inside the root is this library's reading].  One
 * streaming pass: the norm is taken alongside the dot products, x * g in f32
 * for either x dtype.  x: device [m,k] (xt); norm_weight: device [k] of the
 * same dtype; both 16-byte aligned.  eps: finite, >= 0 (a zero row with
 * eps == 0 gives NaN).  4-bit formats need k % 32 == 0 (BSQ_ERR_SHAPE).
 * Weight arguments and out as for bsq_qgemm. */
bsq_status bsq_rmsnorm_qgemv(bsq_format fmt, int block, int64_t m, int64_t n, int64_t k, const void *codes,
                             const void *scales, const void *biases, float global_scale, const void *x,
                             const void *norm_weight, float eps, bsq_dtype xt, void *out, bsq_dtype ot,
                             void *stream);

/* Expert-routed GEMV rows (MoE gather): out[i,j] = sum_p x[i,p] *
 * dequant(W)[expert_ids[i]*n + j, p] for a stack of num_experts experts packed
 * as ONE [num_experts*n, k] weight (layouts as above; nvfp4's global is shared
 * by all experts) [metaltile PR #250, commit adding the per-token
 * expert-routed qmm: the weight row is expert_ids[m]*out_dim + n].  Each
 * routed row streams its own expert's rows (the decode form: one row per
 * token and chosen expert).  expert_ids: device int32 [m], 4-byte aligned;
 * x: device [m,k] (xt), 16-byte aligned; out: device [m,n] (ot).  m <= 65535
 * (BSQ_ERR_SHAPE).  An id outside [0, num_experts) cannot be reported
 * synchronously: that output row is written as zeros and, if status_dev
 * (device int, caller-initialised) is given, it is set to BSQ_ERR_ARG. */
bsq_status bsq_gather_qmm(bsq_format fmt, int block, int64_t m, int64_t n, int64_t k, int64_t num_experts,
                          const void *codes, const void *scales, const void *biases, float global_scale,
                          const int32_t *expert_ids, const void *x, bsq_dtype xt, void *out, bsq_dtype ot,
                          int *status_dev, void *stream);

/* Expert-grouped quantized matmul (prefill-scale MoE): the routed gather's
 * result, out[i,j] = sum_p x[i,p] * dequant(W)[expert_ids[i]*n + j, p], over a
 * stack of num_experts experts packed as ONE [num_experts*n, k] weight
 * [metaltile PR #250, commit adding the per-token expert-routed qmm (the
 * weight row is expert_ids[m]*out_dim + n); rlx-cpu quant.rs,
 * lowp_scaled_grouped_matmul (the expert-indexed GEMM)], computed with the
 * rows grouped by expert: a routing pass on the device sorts the rows by
 * expert into a table in `workspace`, then the bf16 MFMA kernel runs 128-row
 * tiles of each expert's rows; for decode-sized m <= 32 (and a stacked
 * weight under 2 GiB of codes) the decode GEMV kernel routes the rows itself
 * (the workspace is not touched) and runs tiles of up to 4 rows of one
 * expert.  Either way each expert's
 * weight is streamed once per tile instead of once per row.  x: device bf16
 * [m,k], 16-byte aligned (bf16 only).  expert_ids: device int32 [m].  out:
 * device [m,n] (ot).
 * 1 <= num_experts <= 1024, m <= 2^24 (BSQ_ERR_SHAPE otherwise); 4-bit formats
 * need k % 32 == 0 (BSQ_ERR_SHAPE).  workspace: device memory of at least
 * bsq_grouped_qgemm_workspace(m, num_experts) bytes, 4-byte aligned, owned by
 * the caller; its contents on entry do not matter and it must not be shared by
 * calls in flight at the same time.  An id outside [0, num_experts) gives a
 * zero output row and, if status_dev (device int, caller-initialised) is
 * given, sets it to BSQ_ERR_ARG.  Asynchronous on stream. */
bsq_status bsq_grouped_qgemm_workspace(int64_t m, int64_t num_experts, size_t *bytes);
bsq_status bsq_grouped_qgemm(bsq_format fmt, int block, int64_t m, int64_t n, int64_t k, int64_t num_experts,
                             const void *codes, const void *scales, const void *biases, float global_scale,
                             const int32_t *expert_ids, const void *x, void *out, bsq_dtype ot, void *workspace,
                             size_t workspace_bytes, int *status_dev, void *stream);

/* bsq_grouped_qgemm without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, result, checks and errors as bsq_grouped_qgemm; the routing
 * table lives in a 1 MiB array the library keeps on each device until the
 * process ends, so m and num_experts must satisfy
 * bsq_grouped_qgemm_workspace(m, num_experts) <= 1 MiB (any m <= 253000 fits,
 * whatever num_experts; BSQ_ERR_SHAPE otherwise).  Calls on one device share
 * that array: two such calls in flight at once on one device (on different
 * streams, or from different threads) race and give wrong results. */
bsq_status bsq_grouped_qgemm_noalloc(bsq_format fmt, int block, int64_t m, int64_t n, int64_t k, int64_t num_experts,
                                     const void *codes, const void *scales, const void *biases, float global_scale,
                                     const int32_t *expert_ids, const void *x, void *out, bsq_dtype ot,
                                     int *status_dev, void *stream);

/* Calibration (measurement only; not a step of the hot path).  A streaming
 * read of `bytes` bytes of the device buffer `buf` with the decode kernel's
 * load form (one 16-byte nontemporal load per lane, each byte read once,
 * nothing kept): the bandwidth a weight stream of that size reaches on this
 * device, the measured denominator beside the vendor HBM figure.  buf 16-byte
 * aligned, bytes >= 0 and a multiple of 16 (BSQ_ERR_ALIGN / BSQ_ERR_SHAPE);
 * sink: device float, written only for data whose four words XOR to one
 * fixed constant (so the loads cannot be dropped).  Asynchronous on stream. */
bsq_status bsq_calib_read(const void *buf, int64_t bytes, float *sink, void *stream);

/* Calibration: `workgroups` workgroups of 4 waves; each wave runs `iters`
 * steps of four independent v_mfma_f32_32x32x16_bf16 on register operands
 * (no memory traffic).  Work = workgroups * 4 * iters * 4 * 32768 flops; the
 * bf16 matrix-core rate this device sustains, beside the vendor figure.
 * iters >= 0, 1 <= workgroups < 2^31 (BSQ_ERR_ARG); sink: device float.
 * Asynchronous on stream. */
bsq_status bsq_calib_mfma(int64_t iters, int64_t workgroups, float *sink, void *stream);

/* Static text for a status code. */
const char *bsq_status_string(bsq_status s);

/* Detail of the last failing call on this thread ("" if none). */
const char *bsq_last_error(void);

/* Library version string. */
const char *bsq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSQ_H */
