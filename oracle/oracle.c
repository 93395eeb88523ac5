/*
 * oracle.c -- plain, slow, CPU oracle for block-scaled dequantize-and-multiply.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path loads, links or calls
 * this file.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline leg may use it.  It shares no code, header, table or constant with
 * the HIP library; the two meet only through the seeded input generators and
 * the stored byte layouts.
 *
 * What it computes (each step cites the page it follows):
 *   pack     f32 weight [n,k] -> per-block scale + element codes, the codes
 *            quantized against the scale as stored (the "effective" scale)
 *            [metaltile PR #250, commit "QFormat {Nvfp4, Mxfp4, Mxfp8E4, ...}
 *            with pack() and dequant()"; rlx-cpu quant.rs, lowp_compute_scales
 *            and lowp_quantize].
 *   dequant  codes + scales -> f32 [n,k], one rounding to f32 per element
 *            [PR #250, commit "First spec-conformant block-scaled dequant
 *            kernel"; rlx-cpu quant.rs, lowp_dequantize].
 *   matmul   ref[i,j] = sum_p X[i,p] * Wd[j,p] in fp64, with
 *            den[i,j] = sum_p |X[i,p] * Wd[j,p]| alongside (the
 *            dequantize-then-dot reference of PR #250's qgemv / qmm commits).
 *   rmsnorm  Xhat[i,p] = X[i,p] * g[p] / sqrt(mean_p X[i,p]^2 + eps), the
 *            activation of the fused RMSNorm + dequantizing GEMV [PR #250,
 *            commit adding the block-scaled fused RMSNorm + GEMV].
 *   gather   ref[i,j] = sum_p X[i,p] * Wd[e_i * n + j, p] for an expert stack
 *            Wd [E*n, k] and one expert id e_i per row (the expert-routed
 *            gather qmm of PR #250's MoE commit).
 *
 * All arithmetic is fp64 unless a step fixes a stored precision (f32 scales,
 * bf16 int4 scale/bias).  Readings taken where the pages are silent are
 * listed in the header comment of each function.
 *
 * Build: gcc -O2 -std=c99 -fno-fast-math -shared -fPIC -pthread -lm
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Format ids: the numbering is the interface shared with the library's ABI
 * (a stored-layout contract, not shared code). */
enum {
    ORC_MXFP4 = 1,
    ORC_NVFP4 = 2,
    ORC_MXFP8_E4M3 = 3,
    ORC_MXFP8_E5M2 = 4,
    ORC_NVFP8 = 5,
    ORC_INT4_AFFINE = 6,
    ORC_INT8_SYM = 7
};

enum { ORC_OK = 0, ORC_ERR_ARG = 1, ORC_ERR_UNSUPPORTED = 2, ORC_ERR_SHAPE = 3, ORC_ERR_NONFINITE = 5 };

/* ------------------------------------------------------------------------ */
/* Element decoders: code -> exact value (fp64).                             */
/* ------------------------------------------------------------------------ */

/* E2M1: [sign:1][exp:2][mantissa:1].  exp 0 is subnormal with magnitude
 * mantissa/2; otherwise (1 + mantissa/2) * 2^(exp-1).  Levels
 * {0, .5, 1, 1.5, 2, 3, 4, 6} [metaltile-std fp_quantized_mma.rs, module doc
 * "fp4 E2M1 codebook"; PR #250, codec commit].  Code 8 is -0. */
double orc_e2m1_value(unsigned c)
{
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E4M3: [sign:1][exp:4][mantissa:3], bias 7.  exp 0 is subnormal,
 * 2^-6 * m/8; otherwise 2^(exp-7) * (1 + m/8) [fp_quantized_mma.rs, module doc
 * "fp8 E4M3 dequant"].  Reading (the pages disagree on exponent 15): the
 * saturating "no inf" variant of PR #250's codec commit, so exponent 15 is an
 * ordinary binade and only mantissa 7 there is NaN; the largest finite value
 * is 448. */
double orc_e4m3_value(unsigned c)
{
    int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* E5M2: the high byte of an IEEE binary16 [PR #250, codec commit], i.e.
 * bias 15, subnormal m/4 * 2^-14, exponent 31 is inf (m = 0) or NaN
 * [rlx-cpu quant.rs, fp8_e5m2_to_f32]. */
double orc_e5m2_value(unsigned c)
{
    int s = (c >> 7) & 1, e = (c >> 2) & 31, m = c & 3;
    double mag;
    if (e == 31)
        mag = (m == 0) ? INFINITY : NAN;
    else
        mag = (e == 0) ? ldexp((double)m / 4.0, -14) : ldexp(1.0 + m / 4.0, e - 15);
    return s ? -mag : mag;
}

/* E8M0 block scale: 2^(bits-127) [PR #250, codec commit].  Reading: byte 255
 * is NaN (OCP MX), byte 0 is 2^-127. */
double orc_e8m0_value(unsigned b)
{
    return (b == 255) ? NAN : ldexp(1.0, (int)b - 127);
}

/* ------------------------------------------------------------------------ */
/* Rounding to a binary grid.                                                */
/* ------------------------------------------------------------------------ */

/* Round v to the nearest value of a binary float format with `mbits` stored
 * mantissa bits and smallest normal exponent `emin` (subnormals included),
 * ties to even; magnitudes above `maxval` clamp to `maxval`.  Within one
 * binade the grid spacing is 2^(e - mbits); below 2^emin it stays at
 * 2^(emin - mbits).  Dividing by that power of two is exact in fp64 and
 * nearbyint() rounds half to even in the default rounding mode. */
static double round_to_format(double v, int mbits, int emin, double maxval)
{
    double a = fabs(v);
    if (a == 0.0) return v;
    int e = ilogb(a);
    if (e < emin) e = emin;
    double q = ldexp(1.0, e - mbits);
    double r = nearbyint(a / q) * q;
    if (r > maxval) r = maxval;
    return copysign(r, v);
}

/* Element encoders: round the exact quotient to the element grid (ties to
 * even, saturating at the largest finite magnitude) and return the code whose
 * decoded value is that grid point.  The sign bit follows the sign of v, so a
 * negative input that rounds to zero gives the -0 code.  ("midpoint-threshold
 * encode", E4M3 "+-448 saturation, no inf", E5M2 encode "saturates finite
 * inputs" [PR #250, codec commits].) */
unsigned orc_e2m1_encode(double v)
{
    double r = fabs(round_to_format(v, 1, 0, 6.0));
    unsigned sign = signbit(v) ? 8u : 0u;
    for (unsigned c = 0; c < 8; c++)
        if (orc_e2m1_value(c) == r) return c | sign;
    return 0xFFu; /* unreachable for finite v */
}

unsigned orc_e4m3_encode(double v)
{
    double r = fabs(round_to_format(v, 3, -6, 448.0));
    unsigned sign = signbit(v) ? 0x80u : 0u;
    for (unsigned c = 0; c < 0x7F; c++)
        if (orc_e4m3_value(c) == r) return c | sign;
    return 0xFFFu;
}

unsigned orc_e5m2_encode(double v)
{
    double r = fabs(round_to_format(v, 2, -14, 57344.0));
    unsigned sign = signbit(v) ? 0x80u : 0u;
    for (unsigned c = 0; c < 0x7C; c++)
        if (orc_e5m2_value(c) == r) return c | sign;
    return 0xFFFu;
}

/* f64 -> bf16 bits, round to nearest even; overflow goes to inf. */
uint16_t orc_bf16_bits(double v)
{
    double r = round_to_format(v, 7, -126, INFINITY);
    if (fabs(r) > ldexp(2.0 - ldexp(1.0, -7), 127)) r = copysign(INFINITY, v);
    float f = (float)r; /* exact: r is on the bf16 grid */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

double orc_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Format table.                                                             */
/* ------------------------------------------------------------------------ */

/* Block sizes along k: 32 for the MX formats [PR #250 format table],
 * 16 for nvfp4/nvfp8, 64 for int4 affine groups [metaltile-std
 * qmm_gpu_correctness.rs, group_size 64], 32 for int8 blocks. */
int orc_block(int fmt)
{
    switch (fmt) {
    case ORC_MXFP4: case ORC_MXFP8_E4M3: case ORC_MXFP8_E5M2: case ORC_INT8_SYM: return 32;
    case ORC_NVFP4: case ORC_NVFP8: return 16;
    case ORC_INT4_AFFINE: return 64;
    default: return 0;
    }
}

static int is_4bit(int fmt) { return fmt == ORC_MXFP4 || fmt == ORC_NVFP4 || fmt == ORC_INT4_AFFINE; }

/* Stored sizes: 4-bit codes 8 per u32 word along k ([n, k/8] words); 8-bit
 * codes one byte each ([n,k]); scales [n, k/block] as u8 (E8M0, E4M3), f32
 * (nvfp8, int8) or bf16 (int4 scale and bias). */
int orc_sizes(int fmt, int64_t n, int64_t k, int64_t *code_bytes, int64_t *scale_bytes, int64_t *bias_bytes)
{
    int B = orc_block(fmt);
    if (!B) return ORC_ERR_UNSUPPORTED;
    if (n < 0 || k < 0) return ORC_ERR_ARG;
    if (k % B) return ORC_ERR_SHAPE;
    int64_t nb = n * (k / B);
    *code_bytes = is_4bit(fmt) ? n * k / 2 : n * k;
    switch (fmt) {
    case ORC_MXFP4: case ORC_NVFP4: case ORC_MXFP8_E4M3: case ORC_MXFP8_E5M2: *scale_bytes = nb; break;
    case ORC_NVFP8: case ORC_INT8_SYM: *scale_bytes = 4 * nb; break;
    case ORC_INT4_AFFINE: *scale_bytes = 2 * nb; break;
    }
    *bias_bytes = (fmt == ORC_INT4_AFFINE) ? 2 * nb : 0;
    return ORC_OK;
}

/* Code storage helpers: element (j,p) of a 4-bit [n,k] matrix sits in word
 * j*(k/8) + p/8 at bits 4*(p%8).. (low nibble = even element, LSB first)
 * [fp_quantized_mma.rs, "W coop-dequant" step; qmm_gpu_correctness.rs,
 * cpu_qmm_reference]. */
static unsigned get_code(int fmt, const void *codes, int64_t k, int64_t j, int64_t p)
{
    if (is_4bit(fmt)) {
        const uint32_t *w = (const uint32_t *)codes;
        return (w[j * (k / 8) + p / 8] >> (4 * (p % 8))) & 0xFu;
    }
    return ((const uint8_t *)codes)[j * k + p];
}

static void put_code(int fmt, void *codes, int64_t k, int64_t j, int64_t p, unsigned c)
{
    if (is_4bit(fmt)) {
        uint32_t *w = (uint32_t *)codes;
        int64_t idx = j * (k / 8) + p / 8;
        int sh = 4 * (int)(p % 8);
        w[idx] = (w[idx] & ~(0xFu << sh)) | ((uint32_t)(c & 0xFu) << sh);
    } else {
        ((uint8_t *)codes)[j * k + p] = (uint8_t)c;
    }
}

/* ------------------------------------------------------------------------ */
/* Pack.                                                                     */
/* ------------------------------------------------------------------------ */

/* Scale byte for an MX block: OCP shared-exponent rule, floor(log2(amax))
 * minus the element's largest exponent (2 for E2M1, 8 for E4M3, 15 for E5M2),
 * clamped to the E8M0 range; an all-zero block gets 2^0 (rlx-cpu quant.rs,
 * lowp_compute_scales: scale 1.0 when amax is zero). */
static unsigned mx_scale_byte(double amax, int elem_emax)
{
    if (amax == 0.0) return 127;
    int e = ilogb(amax) - elem_emax;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return (unsigned)(e + 127);
}

static unsigned encode_elem(int fmt, double v)
{
    switch (fmt) {
    case ORC_MXFP4: case ORC_NVFP4: return orc_e2m1_encode(v);
    case ORC_MXFP8_E4M3: case ORC_NVFP8: return orc_e4m3_encode(v);
    case ORC_MXFP8_E5M2: return orc_e5m2_encode(v);
    }
    return 0;
}

static double decode_elem(int fmt, unsigned c)
{
    switch (fmt) {
    case ORC_MXFP4: case ORC_NVFP4: return orc_e2m1_value(c);
    case ORC_MXFP8_E4M3: case ORC_NVFP8: return orc_e4m3_value(c);
    case ORC_MXFP8_E5M2: return orc_e5m2_value(c);
    case ORC_INT4_AFFINE: return (double)(c & 0xF);
    case ORC_INT8_SYM: return (double)(int8_t)(uint8_t)c;
    }
    return NAN;
}

/* Pack w (host f32 [n,k], row-major) into codes/scales/biases.
 *   mxfp4/mxfp8: E8M0 per 32-block, codes against 2^(byte-127).
 *   nvfp4: global g = f32(T / (6*448)) from the tensor amax T (1.0 if that is
 *          zero), E4M3 micro code = encode(amax_b / (6 g)) (0x38 = 1.0 for a
 *          zero block), effective scale e4m3(micro) * g ("two-level global FP32
 *          so its E4M3 micro-scales fit +-448", PR #250).
 *   nvfp8: f32 scale f32(amax_b / 448) per 16-block (1.0 for a zero block).
 *   int8:  f32 scale f32(amax_b / 127) per 32-block, q = clamp(rne(w/s), +-127)
 *          (symmetric, +-127 [PR #250, int8 codec commit]).
 *   int4:  per 64-group s = bf16((max-min)/15), b = bf16(min),
 *          q = clamp(rne((w-b)/s), 0, 15); value s*q + b [qmm_gpu_correctness.rs,
 *          cpu_qmm_reference; groups quantized by their min and max].
 * Every code is chosen against the scale exactly as stored; a zero effective
 * scale gives code 0 (rlx-cpu quant.rs, lowp_quantize).  Quotients are formed
 * in fp64.  Non-finite input is rejected. */
int orc_pack(int fmt, const float *w, int64_t n, int64_t k, void *codes, void *scales, void *biases,
             float *global_out)
{
    int B = orc_block(fmt);
    if (!B) return ORC_ERR_UNSUPPORTED;
    if (n < 0 || k < 0) return ORC_ERR_ARG;
    if (k % B) return ORC_ERR_SHAPE;
    for (int64_t i = 0; i < n * k; i++)
        if (!isfinite(w[i])) return ORC_ERR_NONFINITE;
    int64_t nblk = k / B;
    if (is_4bit(fmt)) memset(codes, 0, (size_t)(n * k / 2));

    float g = 1.0f;
    if (fmt == ORC_NVFP4) {
        float T = 0.0f;
        for (int64_t i = 0; i < n * k; i++)
            if (fabsf(w[i]) > T) T = fabsf(w[i]);
        g = T / 2688.0f; /* 2688 = 6 * 448, one f32 rounding */
        if (!(g > 0.0f)) g = 1.0f;
    }
    if (global_out) *global_out = (fmt == ORC_NVFP4) ? g : 1.0f;

    for (int64_t j = 0; j < n; j++) {
        for (int64_t b = 0; b < nblk; b++) {
            const float *blk = w + j * k + b * B;
            int64_t p0 = b * B;
            double amax = 0.0, mn = blk[0], mx = blk[0];
            for (int i = 0; i < B; i++) {
                double a = fabs((double)blk[i]);
                if (a > amax) amax = a;
                if (blk[i] < mn) mn = blk[i];
                if (blk[i] > mx) mx = blk[i];
            }
            double S; /* effective scale, exact in fp64 */
            switch (fmt) {
            case ORC_MXFP4: case ORC_MXFP8_E4M3: case ORC_MXFP8_E5M2: {
                int emax = (fmt == ORC_MXFP4) ? 2 : (fmt == ORC_MXFP8_E4M3) ? 8 : 15;
                unsigned byte = mx_scale_byte(amax, emax);
                ((uint8_t *)scales)[j * nblk + b] = (uint8_t)byte;
                S = orc_e8m0_value(byte);
                for (int i = 0; i < B; i++) put_code(fmt, codes, k, j, p0 + i, encode_elem(fmt, blk[i] / S));
                break;
            }
            case ORC_NVFP4: {
                unsigned micro = (amax == 0.0) ? 0x38u : orc_e4m3_encode(amax / (6.0 * (double)g));
                ((uint8_t *)scales)[j * nblk + b] = (uint8_t)micro;
                S = orc_e4m3_value(micro) * (double)g;
                for (int i = 0; i < B; i++)
                    put_code(fmt, codes, k, j, p0 + i, (S != 0.0) ? orc_e2m1_encode(blk[i] / S) : 0u);
                break;
            }
            case ORC_NVFP8: {
                float s = (amax == 0.0) ? 1.0f : (float)amax / 448.0f;
                ((float *)scales)[j * nblk + b] = s;
                S = s;
                for (int i = 0; i < B; i++)
                    put_code(fmt, codes, k, j, p0 + i, (S != 0.0) ? orc_e4m3_encode(blk[i] / S) : 0u);
                break;
            }
            case ORC_INT8_SYM: {
                float s = (amax == 0.0) ? 1.0f : (float)amax / 127.0f;
                ((float *)scales)[j * nblk + b] = s;
                S = s;
                for (int i = 0; i < B; i++) {
                    double q = 0.0;
                    if (S != 0.0) {
                        q = nearbyint(blk[i] / S);
                        if (q > 127) q = 127;
                        if (q < -127) q = -127;
                    }
                    put_code(fmt, codes, k, j, p0 + i, (unsigned)(uint8_t)(int8_t)q);
                }
                break;
            }
            case ORC_INT4_AFFINE: {
                uint16_t sb = orc_bf16_bits((mx - mn) / 15.0);
                uint16_t bb = orc_bf16_bits(mn);
                ((uint16_t *)scales)[j * nblk + b] = sb;
                ((uint16_t *)biases)[j * nblk + b] = bb;
                double s = orc_bf16_value(sb), bias = orc_bf16_value(bb);
                for (int i = 0; i < B; i++) {
                    double q = 0.0;
                    if (s != 0.0) {
                        q = nearbyint(((double)blk[i] - bias) / s);
                        if (q > 15) q = 15;
                        if (q < 0) q = 0;
                    }
                    put_code(fmt, codes, k, j, p0 + i, (unsigned)q);
                }
                break;
            }
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Dequant.                                                                  */
/* ------------------------------------------------------------------------ */

/* Value of the stored per-block scale as an exact fp64 number. */
static double scale_value(int fmt, const void *scales, int64_t idx)
{
    switch (fmt) {
    case ORC_MXFP4: case ORC_MXFP8_E4M3: case ORC_MXFP8_E5M2:
        return orc_e8m0_value(((const uint8_t *)scales)[idx]);
    case ORC_NVFP4: return orc_e4m3_value(((const uint8_t *)scales)[idx]);
    case ORC_NVFP8: case ORC_INT8_SYM: return (double)((const float *)scales)[idx];
    case ORC_INT4_AFFINE: return orc_bf16_value(((const uint16_t *)scales)[idx]);
    }
    return NAN;
}

/* out[j,p] = f32(decode(code) * scale) with exactly one rounding to f32:
 *   mx:    elem * 2^(byte-127)
 *   nvfp4: (e2m1 * e4m3_micro) * g  (the inner product is exact)
 *   nvfp8: e4m3 * s;  int8: q * s;  int4: s*q + b.
 * Every product and sum here is exact in fp64 for these operand widths, so
 * the single (float) conversion is the only rounding.
 * [PR #250, dequant kernel commits; rlx-cpu quant.rs, lowp_dequantize;
 * qmm_gpu_correctness.rs, int4 "s*q + bias"]. */
int orc_dequant(int fmt, int64_t n, int64_t k, const void *codes, const void *scales, const void *biases,
                float global, float *out)
{
    int B = orc_block(fmt);
    if (!B) return ORC_ERR_UNSUPPORTED;
    if (n < 0 || k < 0) return ORC_ERR_ARG;
    if (k % B) return ORC_ERR_SHAPE;
    int64_t nblk = k / B;
    for (int64_t j = 0; j < n; j++) {
        for (int64_t p = 0; p < k; p++) {
            unsigned c = get_code(fmt, codes, k, j, p);
            double e = decode_elem(fmt, c);
            double s = scale_value(fmt, scales, j * nblk + p / B);
            double v;
            if (fmt == ORC_INT4_AFFINE)
                v = s * e + orc_bf16_value(((const uint16_t *)biases)[j * nblk + p / B]);
            else if (fmt == ORC_NVFP4)
                v = (e * s) * (double)global;
            else
                v = e * s;
            out[j * k + p] = (float)v;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Matmul in fp64.                                                           */
/* ------------------------------------------------------------------------ */

struct mm_job {
    const float *x, *wd;
    const double *xd; /* fp64 X instead of x when not NULL */
    const int64_t *rows;
    int64_t nrows, n, k, r0, r1;
    double *ref, *den;
};

static void *mm_worker(void *arg)
{
    struct mm_job *J = (struct mm_job *)arg;
    for (int64_t r = J->r0; r < J->r1; r++) {
        const float *xr = J->xd ? NULL : J->x + J->rows[r] * J->k;
        const double *xdr = J->xd ? J->xd + J->rows[r] * J->k : NULL;
        for (int64_t j = 0; j < J->n; j++) {
            const float *wr = J->wd + j * J->k;
            double acc = 0.0, mag = 0.0;
            for (int64_t p = 0; p < J->k; p++) {
                double t = (xdr ? xdr[p] : (double)xr[p]) * (double)wr[p];
                acc += t;
                mag += fabs(t);
            }
            J->ref[r * J->n + j] = acc;
            J->den[r * J->n + j] = mag;
        }
    }
    return NULL;
}

/* For each listed row i of X (f32 [m,k]; bf16 inputs are passed as their
 * exact f32 values) and every j < n:
 *   ref[r,j] = sum_p X[i,p] * Wd[j,p],  den[r,j] = sum_p |X[i,p] * Wd[j,p]|,
 * summed in order of p in fp64.  `rows` may be NULL for all m rows.  Rows
 * are split statically over `threads` workers (no change to any sum). */
static int matmul_any(const float *x, const double *xd, const float *wd, int64_t m, int64_t n, int64_t k,
                      const int64_t *rows, int64_t nrows, double *ref, double *den, int threads)
{
    if (m < 0 || n < 0 || k < 0) return ORC_ERR_ARG;
    int64_t *all = NULL;
    if (!rows) {
        all = (int64_t *)malloc(sizeof(int64_t) * (size_t)(m > 0 ? m : 1));
        for (int64_t i = 0; i < m; i++) all[i] = i;
        rows = all;
        nrows = m;
    }
    for (int64_t r = 0; r < nrows; r++)
        if (rows[r] < 0 || rows[r] >= m) {
            free(all);
            return ORC_ERR_ARG;
        }
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    if (threads > nrows) threads = (int)(nrows > 0 ? nrows : 1);
    pthread_t tid[256];
    struct mm_job jobs[256];
    int64_t per = (nrows + threads - 1) / threads;
    for (int t = 0; t < threads; t++) {
        int64_t r0 = t * per, r1 = r0 + per;
        if (r0 > nrows) r0 = nrows;
        if (r1 > nrows) r1 = nrows;
        jobs[t] = (struct mm_job){x, wd, xd, rows, nrows, n, k, r0, r1, ref, den};
        if (threads == 1)
            mm_worker(&jobs[t]);
        else
            pthread_create(&tid[t], NULL, mm_worker, &jobs[t]);
    }
    if (threads > 1)
        for (int t = 0; t < threads; t++) pthread_join(tid[t], NULL);
    free(all);
    return ORC_OK;
}

int orc_matmul(const float *x, const float *wd, int64_t m, int64_t n, int64_t k, const int64_t *rows,
               int64_t nrows, double *ref, double *den, int threads)
{
    return matmul_any(x, NULL, wd, m, n, k, rows, nrows, ref, den, threads);
}

/* orc_matmul with an fp64 X [m,k] (used for the normalized activation). */
int orc_matmul_f64(const double *x, const float *wd, int64_t m, int64_t n, int64_t k, const int64_t *rows,
                   int64_t nrows, double *ref, double *den, int threads)
{
    return matmul_any(NULL, x, wd, m, n, k, rows, nrows, ref, den, threads);
}

/* ------------------------------------------------------------------------ */
/* RMSNorm of the activation (fused RMSNorm + dequantizing GEMV).            */
/* ------------------------------------------------------------------------ */

/* Xhat[i,p] = X[i,p] * g[p] * r_i,  r_i = 1 / sqrt((sum_p X[i,p]^2) / k + eps),
 * in fp64.  The pages describe the fused op as a first phase that sums x^2
 * into the row's inverse RMS and a second that accumulates the GEMV over
 * x * norm_weight * inv_rms [metaltile PR #250, commit adding the block-scaled
 * fused RMSNorm + dequantizing GEMV]; they print no formula for the inverse
 * RMS, so the usual one is the reading taken: the mean of squares over the k
 * elements of the row, eps added inside the square root.  X is [m,k] f32 (bf16
 * inputs as their exact f32 values), g is [k] f32, Xhat is fp64 [m,k].
 * k == 0 leaves Xhat empty; eps must be >= 0 and the row must not be all zero
 * when eps == 0 (ORC_ERR_ARG otherwise). */
int orc_rmsnorm(const float *x, const float *g, int64_t m, int64_t k, double eps, double *xhat)
{
    if (m < 0 || k < 0 || !(eps >= 0.0)) return ORC_ERR_ARG;
    for (int64_t i = 0; i < m; i++) {
        const float *xr = x + i * k;
        double ss = 0.0;
        for (int64_t p = 0; p < k; p++) ss += (double)xr[p] * (double)xr[p];
        if (k == 0) continue;
        const double ms = ss / (double)k + eps;
        if (!(ms > 0.0)) return ORC_ERR_ARG;
        const double r = 1.0 / sqrt(ms);
        for (int64_t p = 0; p < k; p++) xhat[i * k + p] = (double)xr[p] * (double)g[p] * r;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Expert-routed matmul (MoE gather).                                        */
/* ------------------------------------------------------------------------ */

/* ref[i,j] = sum_p X[i,p] * Wd[ids[i]*n + j, p] and den[i,j] = sum_p |...| in
 * fp64, p in order, for X f32 [m,k] and the dequantized expert stack Wd f32
 * [E*n, k] [metaltile PR #250, commit adding the per-token expert-routed
 * matmul: output[m,n] = sum_k dequant(weight[expert_ids[m], n, k]) * x[m,k],
 * the stack stored as one [E*out_dim, in_dim] tensor so the weight row is
 * expert_ids[m]*out_dim + n].  An id outside [0, E) is an argument error. */
int orc_gather_matmul(const float *x, const float *wd, const int32_t *ids, int64_t m, int64_t n, int64_t k,
                      int64_t E, double *ref, double *den)
{
    if (m < 0 || n < 0 || k < 0 || E < 1) return ORC_ERR_ARG;
    for (int64_t i = 0; i < m; i++)
        if (ids[i] < 0 || ids[i] >= E) return ORC_ERR_ARG;
    for (int64_t i = 0; i < m; i++) {
        const float *xr = x + i * k;
        for (int64_t j = 0; j < n; j++) {
            const float *wr = wd + ((int64_t)ids[i] * n + j) * k;
            double acc = 0.0, mag = 0.0;
            for (int64_t p = 0; p < k; p++) {
                const double t = (double)xr[p] * (double)wr[p];
                acc += t;
                mag += fabs(t);
            }
            ref[i * n + j] = acc;
            den[i * n + j] = mag;
        }
    }
    return ORC_OK;
}
