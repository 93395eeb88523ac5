"""GPU parity at the edges: every kernel instantiation the library can pick,
extreme scale encodings, ragged and multi-round k, and the prefill workloads
checked on every output row.

Same bar as test_gpu_parity: |gpu - ref| <= tol * sum_p |x_p * w_p| with the
oracle's fp64 dequant-then-dot as ref; NaN where the oracle gives NaN.
"""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_bit_e2m1_amd import bsq, workloads
from tests.test_gpu_parity import (ALL, BLOCK, DEV, MX_TOL, _mx_case, _exact_mx_codes, check_bound, packed,
                                   raw_weight)

pytestmark = pytest.mark.gpu

MX = ["mxfp4", "mxfp8_e4m3", "mxfp8_e5m2"]
THREADS = 16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsq.lib()
    oracle.lib()
    yield
    torch.cuda.synchronize()


def _x(m, k, seed, act, scale=1.0):
    X = (np.random.default_rng(seed).standard_normal((m, k)) * scale).astype(np.float32)
    if act == "bf16":
        X = torch.from_numpy(X).to(torch.bfloat16).float().numpy()
    return X


def _run(d, X, act, path, out_dtype=None):
    xt = torch.from_numpy(X).to(torch.bfloat16 if act == "bf16" else torch.float32).to(DEV)
    od = out_dtype or xt.dtype
    if path == "gemv":
        return bsq.qgemv(d, xt[0], out_dtype=od)[None, :].float().cpu().numpy(), od == torch.bfloat16
    return bsq.qgemm(d, xt, out_dtype=od, path=path).float().cpu().numpy(), od == torch.bfloat16


def _check(out, ref, den, tol, what, bf16_out):
    nan = np.isnan(ref)
    assert (np.isnan(out) == nan).all(), f"{what}: NaN pattern differs ({int((np.isnan(out) != nan).sum())} outputs)"
    check_bound(np.where(nan, 0.0, out), np.where(nan, 0.0, ref), np.where(nan, 0.0, den), tol, what, bf16_out)


# ----------------------------------------------------------------- ragged and multi-round k
@pytest.mark.parametrize("k", [2064, 4112])
def test_nvfp4_ragged_k_past_the_first_round(k):
    """nvfp4 with k % 32 == 16: the code rows are not 16-byte aligned, so the
    streaming kernel reads them word by word in guarded rounds; every round up
    to k must run (qgemv, rows qgemm, routed gather; bf16 and f32 x)."""
    n = 45
    W = workloads.random_weights(n, k, seed=k, sigma=0.02)
    p, d = packed("nvfp4", W)
    wd = oracle.dequant_packed(p)
    for act in ("bf16", "f32"):
        tol = 2e-3 if act == "bf16" else 1e-5
        X = _x(3, k, k + 1, act)
        ref, den = oracle.matmul(X, wd)
        out, b = _run(d, X[:1], act, "gemv")
        check_bound(out, ref[:1], den[:1], tol, f"qgemv nvfp4 k={k} {act}", b)
        out, b = _run(d, X, act, bsq.PATH_ROWS)
        check_bound(out, ref, den, tol, f"rows nvfp4 k={k} {act}", b)
        E = 3
        Ws = workloads.random_weights(E * n, k, seed=k + 2, sigma=0.02)
        ps, ds = packed("nvfp4", Ws)
        ids = np.array([2, 0, 2], np.int32)
        rg, dg = oracle.gather_matmul(X, oracle.dequant_packed(ps), ids, n)
        xt = torch.from_numpy(X).to(torch.bfloat16 if act == "bf16" else torch.float32).to(DEV)
        out = bsq.gather_qmm(ds, E, torch.from_numpy(ids).to(DEV), xt).float().cpu().numpy()
        check_bound(out, rg, dg, tol, f"gather nvfp4 k={k} {act}", act == "bf16")


@pytest.mark.parametrize("fmt", ALL)
def test_decode_gemv_several_rounds_and_ragged_n(fmt):
    """The decode GEMV walks k in rounds of 64 chunks per wave of a k split:
    k = 8256 needs two full rounds and a ragged third; n = 37 leaves a partial
    row group; routed rows (gather) take the same kernel."""
    n, k = 37, 8256
    W = workloads.random_weights(n, k, seed=3, sigma=0.02, outliers=True)
    p, d = packed(fmt, W)
    wd = oracle.dequant_packed(p)
    X = _x(1, k, 4, "bf16")
    ref, den = oracle.matmul(X, wd)
    for od in (torch.bfloat16, torch.float32):
        out, b = _run(d, X, "bf16", "gemv", od)
        check_bound(out, ref, den, 2e-3, f"gemv {fmt} k={k} {od}", b)
    E = 2
    Ws = workloads.random_weights(E * n, k, seed=5, sigma=0.02)
    ps, ds = packed(fmt, Ws)
    ids = np.array([1, 1, 0], np.int32)
    X3 = _x(3, k, 6, "bf16")
    rg, dg = oracle.gather_matmul(X3, oracle.dequant_packed(ps), ids, n)
    out = bsq.gather_qmm(ds, E, torch.from_numpy(ids).to(DEV),
                         torch.from_numpy(X3).to(torch.bfloat16).to(DEV)).float().cpu().numpy()
    check_bound(out, rg, dg, 2e-3, f"gather {fmt} k={k}", True)


# ----------------------------------------------------------------- extreme scales
def _mx_codes(fmt, n, k, rng, max_mag_code=None):
    """Random element codes (no NaN codes); max_mag_code keeps magnitudes
    below 2 (E2M1 codes <= 2, E4M3 exponent field <= 7, E5M2 <= 15), so that
    times 2^127 they stay finite in f32 and bf16."""
    if fmt == "mxfp4":
        mag = rng.integers(0, 8 if max_mag_code is None else 3, (n, k))
        nib = ((rng.integers(0, 2, (n, k)) << 3) | mag).astype(np.uint8)
        return np.ascontiguousarray(nib[:, 0::2] | (nib[:, 1::2] << 4)).reshape(-1)
    sign = rng.integers(0, 2, (n, k)) << 7
    if fmt == "mxfp8_e4m3":
        hi = 15 if max_mag_code is None else 8
        e = rng.integers(0, hi, (n, k))
        c = sign | (e << 3) | rng.integers(0, 8, (n, k))
        c = np.where((c & 0x7F) == 0x7F, c ^ 1, c)
    else:
        hi = 31 if max_mag_code is None else 16
        c = sign | (rng.integers(0, hi, (n, k)) << 2) | rng.integers(0, 4, (n, k))
    return np.ascontiguousarray(c.astype(np.uint8)).reshape(-1)


def _extreme_cases(fmt, n, k, rng):
    """(name, codes, scales, x scale): tiny scales (E8M0 bytes 0..8) with some
    ordinary blocks, huge scales (bytes 250..254, element magnitudes below 2
    so every dequantized weight stays finite) with x scaled down so no sum
    overflows, and NaN scales (byte 255) in the last two rows."""
    nb = k // 32
    tiny = np.where(rng.random((n, nb)) < 0.75, rng.integers(0, 9, (n, nb)), rng.integers(118, 128, (n, nb)))
    tiny[: n // 2] = rng.integers(0, 9, (n // 2, nb))  # half the rows hold only tiny blocks
    huge = rng.integers(250, 255, (n, nb))
    nan = rng.integers(110, 130, (n, nb))
    nan[-2:, nb // 2] = 255
    return [("tiny", _mx_codes(fmt, n, k, rng), tiny.astype(np.uint8).reshape(-1), 1.0),
            ("huge", _mx_codes(fmt, n, k, rng, max_mag_code=True), huge.astype(np.uint8).reshape(-1), 2.0 ** -16),
            ("nan", _mx_codes(fmt, n, k, rng), nan.astype(np.uint8).reshape(-1), 1.0)]


@pytest.mark.parametrize("fmt", MX)
def test_e8m0_extreme_bytes_every_kernel(fmt):
    """E8M0 bytes 0..8 (2^-127 is an f32 subnormal), 250..254 and 255 (NaN)
    through the decode GEMV (bf16 x), the streaming kernel (f32 x, and m = 3
    bf16), the bf16 MFMA kernel (whose weight conversion takes the scale byte
    as an exponent-only operand), the grouped decode form (tiles of 4 and 2
    rows) and, as the weight of the scaled MFMA GEMM."""
    rng = np.random.default_rng(77)
    n, k, m = 80, 512, 40
    for name, codes, scales, xs in _extreme_cases(fmt, n, k, rng):
        p, d = raw_weight(fmt, n, k, codes, scales)
        wd = oracle.dequant_packed(p)
        for act in ("bf16", "f32"):
            X = _x(m, k, 9, act, xs)
            ref, den = oracle.matmul(X, wd)
            tol = 2e-3 if act == "bf16" else 1e-5
            out, b = _run(d, X[:1], act, "gemv")
            _check(out, ref[:1], den[:1], tol, f"{fmt} {name} gemv {act}", b)
            out, b = _run(d, X[:3], act, bsq.PATH_ROWS)
            _check(out, ref[:3], den[:3], tol, f"{fmt} {name} rows m=3 {act}", b)
        X = _x(m, k, 9, "bf16", xs)
        ref, den = oracle.matmul(X, wd)
        for od in (torch.float32, torch.bfloat16):
            out, b = _run(d, X, "bf16", bsq.PATH_MFMA, od)
            _check(out, ref, den, 2e-3, f"{fmt} {name} mfma {od}", b)
        # the expert-grouped decode form: the weight as 2 experts of n / 2 rows, tiles of 4 and 2 rows
        ids = np.array([0, 1, 0, 0, 1, 0], np.int32)
        rg, dg = oracle.gather_matmul(X[:6], wd, ids, n // 2)
        xg = torch.from_numpy(X[:6]).to(torch.bfloat16).to(DEV)
        for od in (torch.float32, torch.bfloat16):
            out = bsq.grouped_qmm(d, 2, torch.from_numpy(ids).to(DEV), xg, out_dtype=od).float().cpu().numpy()
            _check(out, rg, dg, 2e-3, f"{fmt} {name} grouped decode form {od}", od == torch.bfloat16)
        # scaled MFMA: X packed with the same MX format (ordinary scales)
        xq = bsq.quantize(fmt, torch.from_numpy(X).to(torch.bfloat16).to(DEV))
        px = oracle.pack(fmt, X)
        r2, d2 = oracle.matmul(oracle.dequant_packed(px), wd)
        for od in (torch.float32, torch.bfloat16):
            out = bsq.qgemm_mx(xq, d, out_dtype=od).float().cpu().numpy()
            _check(out, r2, d2, MX_TOL, f"{fmt} {name} qgemm_mx {od}", od == torch.bfloat16)


def test_nvfp4_every_micro_scale_code_and_extreme_globals():
    """All 256 E4M3 micro-scale codes (one per weight row; 0x7F and 0xFF are
    NaN) through the decode GEMV, the streaming kernel and the MFMA kernel,
    with globals 1, 3e30 and 1e-40 (an f32 subnormal).

    With g = 1e-40 most dequantized weights are f32 subnormals, which the
    oracle's f32 dequant rounds to a multiple of 2^-149, while the kernels
    apply g once to the accumulated sum (as the nvfp4 definition folds the
    global after the dot).  The oracle's own rounding, at most 2^-150 per
    weight, is added to the bound: tol * sum|x*w| + 2^-150 * sum|x|."""
    rng = np.random.default_rng(12)
    n, k = 256, 512
    nib = rng.integers(0, 16, (n, k)).astype(np.uint8)
    codes = np.ascontiguousarray(nib[:, 0::2] | (nib[:, 1::2] << 4)).reshape(-1)
    scales = np.repeat(np.arange(256, dtype=np.uint8), k // 16)
    for g in (1.0, 3.0e30, 1e-40):
        p, d = raw_weight("nvfp4", n, k, codes, scales, g=g)
        wd = oracle.dequant_packed(p)
        for act in ("bf16", "f32"):
            X = _x(16, k, 13, act)
            ref, den = oracle.matmul(X, wd)
            tol = 2e-3 if act == "bf16" else 1e-5
            if g < 1e-38:  # the reference's subnormal rounding, as a term of den
                den = den + (2.0 ** -150 / tol) * np.abs(X.astype(np.float64)).sum(1, keepdims=True)
            out, b = _run(d, X[:1], act, "gemv")
            _check(out, ref[:1], den[:1], tol, f"nvfp4 g={g} gemv {act}", b)
            out, b = _run(d, X[:3], act, bsq.PATH_ROWS)
            _check(out, ref[:3], den[:3], tol, f"nvfp4 g={g} rows {act}", b)
        X = _x(16, k, 13, "bf16")
        ref, den = oracle.matmul(X, wd)
        if g < 1e-38:
            den = den + (2.0 ** -150 / 2e-3) * np.abs(X.astype(np.float64)).sum(1, keepdims=True)
        out, b = _run(d, X, "bf16", bsq.PATH_MFMA, torch.float32)
        _check(out, ref, den, 2e-3, f"nvfp4 g={g} mfma", b)


# ----------------------------------------------------------------- every tile instantiation
@pytest.mark.parametrize("xfmt", MX)
@pytest.mark.parametrize("wfmt", MX)
def test_qgemm_mx_big_tiles(xfmt, wfmt):
    """m = 1024, n = 8192 gives 256 tiles of 256 x 128, the instantiation the
    benchmark times for each operand pair; checked on a seeded sample of rows
    (random data, stated bound) and bit-exact on codes whose sums are exact.
    k = 128 and 512 leave the steady loop empty (the codes are loaded 2-3
    steps ahead: prologue and guarded drain only); k = 2176 (17 steps) runs
    whole 4-step trips and then a 1-step drain."""
    m, n = 1024, 8192
    rng = np.random.default_rng(31)
    rows = np.unique(np.concatenate([[0, 255, 256, m - 1], rng.choice(m, 60, replace=False)]))
    for k, od in ((512, torch.float32), (512, torch.bfloat16), (128, torch.float32), (2176, torch.bfloat16)):
        out, ref, den = _mx_case(xfmt, wfmt, m, n, k, seed=77 + k, out_dtype=od, rows=rows)
        check_bound(out, ref, den, MX_TOL, f"qgemm_mx big tiles {xfmt}x{wfmt} k={k} {od}", od == torch.bfloat16)
    k = 512
    xc, xs = _exact_mx_codes(xfmt, m, k, rng)
    wc, ws = _exact_mx_codes(wfmt, n, k, rng)
    fx, fw = bsq._fmt(xfmt), bsq._fmt(wfmt)
    xd = oracle.dequant(fx, m, k, xc, xs, None, 1.0)
    wd = oracle.dequant(fw, n, k, wc, ws, None, 1.0)
    ref, _ = oracle.matmul(xd, wd, rows=rows, threads=THREADS)
    t = lambda a: torch.from_numpy(a).to(DEV)
    out = bsq.qgemm_mx(bsq.PackedWeight(fx, m, k, t(xc), t(xs), None, 1.0),
                       bsq.PackedWeight(fw, n, k, t(wc), t(ws), None, 1.0), out_dtype=torch.float32)
    out = out.cpu().numpy()[rows].astype(np.float64)
    assert (out == ref).all(), f"{int((out != ref).sum())} inexact outputs"


@pytest.mark.parametrize("fmt", ALL)
def test_mfma_tall_tile(fmt):
    """m = 257, n = 8192 selects the 256 x 128 tile with 2 x 4 waves (fewer
    than 128 tiles of 128 x 256 but at least 128 of 256 x 128): every row,
    bf16 and f32 output."""
    m, n, k = 257, 8192, 512
    W = workloads.random_weights(n, k, seed=90, sigma=0.02, outliers=True)
    p, d = packed(fmt, W)
    X = _x(m, k, 91, "bf16")
    ref, den = oracle.matmul(X, oracle.dequant_packed(p), threads=THREADS)
    for od in (torch.bfloat16, torch.float32):
        out, b = _run(d, X, "bf16", bsq.PATH_MFMA, od)
        check_bound(out, ref, den, 2e-3, f"mfma tall tile {fmt} {od}", b)


# ----------------------------------------------------------------- full prefill workloads
@pytest.mark.parametrize("name", ["mxfp4_qgemm_2048", "int4_affine_qgemm_512", "int8_sym_qgemm_512"])
def test_prefill_workload_every_row(name):
    """The prefill workloads in the benchmark's launch configuration, every
    output row against the oracle (fp64 dot split over host threads)."""
    wl = workloads.WORKLOADS[name]
    W, X = workloads.generate(wl)
    pw = bsq.to_device(bsq.pack(wl.fmt, W), DEV)
    p = oracle.pack(wl.fmt, W)
    assert (p["codes"] == pw.codes.cpu().numpy()).all()
    out = bsq.qgemm(pw, torch.from_numpy(X).to(torch.bfloat16).to(DEV)).float().cpu().numpy()
    ref, den = oracle.matmul(X, oracle.dequant_packed(p), threads=THREADS)
    check_bound(out, ref, den, wl.tol, name, True)
