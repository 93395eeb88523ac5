"""Pins for the oracle's pack, dequant and matmul (CPU only).

Each property is computed here from independent decode tables (torch /
numpy) or from a library routine, never by re-calling the oracle's own
formula:
  * byte-layout sizes of every format;
  * zero blocks get the unit scale and all-zero codes;
  * MX scales follow the shared-exponent rule (amax/S in [2^emax, 2^(emax+1)));
  * every stored code is a nearest grid point to w/S for the stored scale;
  * MX packing is idempotent;
  * nvfp4's two-level scale (global from the tensor amax, E4M3 micro-scale);
  * dequant equals decode(code) * scale with one f32 rounding, also over
    exhaustive code x scale sweeps;
  * the fp64 matmul equals numpy's fp64 matmul and a Python triple loop, and
    the int4 "algebraic split" s*sum(q*x) + b*sum(x) of the int4 reference.
"""
import math

import numpy as np
import pytest
import torch

from block_scaled_bit_e2m1_amd import workloads
from tests.test_oracle_codec import golden_e2m1_table, half_e5m2_table, torch_e4m3_table, torch_e8m0_table

ALL = ["mxfp4", "nvfp4", "mxfp8_e4m3", "mxfp8_e5m2", "nvfp8", "int4_affine", "int8_sym"]
BLOCK = {"mxfp4": 32, "nvfp4": 16, "mxfp8_e4m3": 32, "mxfp8_e5m2": 32, "nvfp8": 16, "int4_affine": 64, "int8_sym": 32}
FOUR_BIT = {"mxfp4", "nvfp4", "int4_affine"}


def codes_of(fmt, p):
    """Unpack stored codes to an [n,k] int array (LSB-first nibbles)."""
    n, k = p["n"], p["k"]
    raw = p["codes"]
    if fmt in FOUR_BIT:
        lo = raw & 0xF
        hi = raw >> 4
        return np.stack([lo, hi], axis=-1).reshape(n, k).astype(np.int64)
    return raw.reshape(n, k).astype(np.int64)


def elem_table(fmt):
    if fmt in ("mxfp4", "nvfp4"):
        return golden_e2m1_table()
    if fmt in ("mxfp8_e4m3", "nvfp8"):
        return torch_e4m3_table()
    if fmt == "mxfp8_e5m2":
        return half_e5m2_table()
    if fmt == "int4_affine":
        return np.arange(16, dtype=np.float64)
    return np.arange(256, dtype=np.uint8).view(np.int8).astype(np.float64)


def bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def scales_f64(fmt, p):
    """Effective per-block scale [n, k/B] in fp64 from independent tables."""
    n, k, B = p["n"], p["k"], BLOCK[fmt]
    s = p["scales"]
    if fmt.startswith("mx"):
        return torch_e8m0_table()[s].reshape(n, k // B)
    if fmt == "nvfp4":
        return torch_e4m3_table()[s].reshape(n, k // B) * np.float64(p["global"])
    if fmt in ("nvfp8", "int8_sym"):
        return s.view(np.float32).astype(np.float64).reshape(n, k // B)
    return bf16_to_f64(s.view(np.uint16)).reshape(n, k // B)


def test_byte_layout_sizes(orc):
    mib = 1 << 20
    assert orc.sizes("mxfp4", 16, 512) == (4096, 256, 0)
    assert orc.sizes("nvfp4", 4096, 4096) == (8 * mib, 1 * mib, 0)
    assert orc.sizes("mxfp8_e4m3", 14336, 4096) == (56 * mib, 14336 * 128, 0)
    assert orc.sizes("mxfp4", 4096, 4096) == (8 * mib, 512 * 1024, 0)
    assert orc.sizes("int4_affine", 11008, 4096) == (11008 * 2048, 11008 * 64 * 2, 11008 * 64 * 2)
    assert orc.sizes("int8_sym", 11008, 4096) == (11008 * 4096, 11008 * 128 * 4, 0)
    assert orc.sizes("nvfp8", 8, 64) == (512, 8 * 4 * 4, 0)
    with pytest.raises(orc.OracleError):
        orc.sizes("mxfp4", 4, 48)  # k not a multiple of the block


@pytest.mark.parametrize("fmt", ALL)
def test_zero_blocks(orc, fmt):
    w = np.zeros((3, 128), dtype=np.float32)
    w[1, 64:] = np.linspace(-1, 1, 64, dtype=np.float32)
    p = orc.pack(fmt, w)
    c = codes_of(fmt, p)
    assert (c[0] == 0).all() and (c[2] == 0).all()
    s = p["scales"]
    if fmt.startswith("mx"):
        assert (s.reshape(3, -1)[0] == 127).all()
    elif fmt == "nvfp4":
        assert (s.reshape(3, -1)[0] == 0x38).all()
    elif fmt in ("nvfp8", "int8_sym"):
        assert (s.view(np.float32).reshape(3, -1)[0] == 1.0).all()
    else:
        assert (s.view(np.uint16).reshape(3, -1)[0] == 0).all()
        assert (p["biases"].view(np.uint16).reshape(3, -1)[0] == 0).all()
    wd = orc.dequant_packed(p)
    assert (wd[0] == 0).all() and (wd[2] == 0).all()


@pytest.mark.parametrize("fmt,emax", [("mxfp4", 2), ("mxfp8_e4m3", 8), ("mxfp8_e5m2", 15)])
def test_mx_shared_exponent_rule(orc, fmt, emax):
    w = workloads.random_weights(64, 256, seed=3, sigma=0.02, outliers=True)
    w[5, :32] *= 1e-30  # tiny block
    w[6, :32] *= 1e30  # huge block
    p = orc.pack(fmt, w)
    S = scales_f64(fmt, p)
    amax = np.abs(w.astype(np.float64)).reshape(64, -1, 32).max(-1)
    r = amax / S
    ok = (r >= 2.0 ** emax) & (r < 2.0 ** (emax + 1))
    assert ok.all()


@pytest.mark.parametrize("fmt", ALL)
def test_codes_are_nearest_for_stored_scale(orc, fmt):
    """Brute force: every code minimizes |dec(c)*S (+b) - w| over all codes."""
    w = workloads.random_weights(24, 256, seed=5, sigma=0.02, outliers=True)
    w[0, :] = np.float32(0.5)  # constant group
    p = orc.pack(fmt, w)
    c = codes_of(fmt, p)
    S = np.repeat(scales_f64(fmt, p), BLOCK[fmt], axis=1)
    table = elem_table(fmt)
    valid = np.array([np.isfinite(t) for t in table])
    if fmt == "int8_sym":
        valid[128] = False  # -128 is never emitted (symmetric +-127)
    cand = table[valid]
    w64 = w.astype(np.float64)
    if fmt == "int4_affine":
        b = np.repeat(bf16_to_f64(p["biases"].view(np.uint16)).reshape(24, -1), 64, axis=1)
        recon = table[c] * S + b
        all_recon = cand[None, None, :] * S[..., None] + b[..., None]
    else:
        recon = table[c] * S
        all_recon = cand[None, None, :] * S[..., None]
    best = np.abs(all_recon - w64[..., None]).min(-1)
    err = np.abs(recon - w64)
    assert (err <= best).all(), np.argwhere(err > best)[:5]


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8_e4m3", "mxfp8_e5m2"])
def test_mx_pack_idempotent(orc, fmt):
    w = workloads.random_weights(32, 512, seed=9, sigma=1.0, outliers=True)
    p = orc.pack(fmt, w)
    p2 = orc.pack(fmt, orc.dequant_packed(p))
    assert (p["codes"] == p2["codes"]).all() and (p["scales"] == p2["scales"]).all()


def test_nvfp4_two_level_scales(orc):
    w = workloads.random_weights(32, 256, seed=21, sigma=0.02)
    p = orc.pack("nvfp4", w)
    T = np.abs(w).max()
    g = np.float32(T) / np.float32(2688.0)
    assert p["global"] == g
    t = torch_e4m3_table()
    amax = np.abs(w.astype(np.float64)).reshape(32, -1, 16).max(-1)
    target = amax / (6.0 * np.float64(g))
    micro = p["scales"].reshape(32, -1)
    finite = np.array([c for c in range(127)])
    for i in range(32):
        for b in range(micro.shape[1]):
            d = np.abs(t[finite] - target[i, b])
            assert abs(t[micro[i, b]] - target[i, b]) == d.min()
    assert (t[micro] <= 448).all()


def test_int4_min_max_rule(orc):
    w = workloads.random_weights(16, 256, seed=22, sigma=0.02)
    p = orc.pack("int4_affine", w)
    g = w.reshape(16, -1, 64)
    mn = g.min(-1)
    b = bf16_to_f64(p["biases"].view(np.uint16)).reshape(16, -1)
    want_b = torch.from_numpy(mn).to(torch.bfloat16).double().numpy()
    assert (b == want_b).all()
    s = bf16_to_f64(p["scales"].view(np.uint16)).reshape(16, -1)
    exact = (g.max(-1).astype(np.float64) - mn.astype(np.float64)) / 15.0
    # s is a bf16 neighbour of the exact quotient, and the nearest one
    up = torch.from_numpy(exact).to(torch.bfloat16).double().numpy()
    assert (s == up).all()


def test_int8_amax_rule(orc):
    w = workloads.random_weights(16, 256, seed=23, sigma=0.02)
    p = orc.pack("int8_sym", w)
    s = p["scales"].view(np.float32).reshape(16, -1)
    amax = np.abs(w).reshape(16, -1, 32).max(-1)
    assert (s == (amax / np.float32(127.0)).astype(np.float32)).all()
    q = codes_of("int8_sym", p).reshape(16, -1, 32)
    q = np.where(q > 127, q - 256, q)
    want = np.clip(np.rint(w.reshape(16, -1, 32).astype(np.float64) / s[..., None].astype(np.float64)), -127, 127)
    assert (q == want).all()
    assert (np.abs(q).max(-1) == 127).all()


def test_nvfp8_amax_rule(orc):
    """nvfp8 keeps one f32 scale per 16-block chosen so the block amax lands on
    E4M3's largest finite value, 448 (format table of metaltile PR #250: nvfp8 is
    E4M3 elements, block 16, FP32 scale; rlx-cpu quant.rs lowp_compute_scales
    divides the amax by the element format's largest finite value).  Pinned
    without the oracle's formula: the top element of every non-zero block must
    take code 0x7E (448 from torch's float8_e4m3fn table, which a 240 maximum
    would miss: its top code would be 0x77) and must reconstruct the amax to
    within f32 rounding (which a 480 maximum would miss: that saturates the top
    element 6.7% low).  The stored scale is also the correctly rounded f32
    quotient, and zero blocks keep scale 1 and all-zero codes."""
    rng = np.random.default_rng(24)
    w = (rng.standard_normal((24, 256)) * 0.02).astype(np.float32)
    w[3, 16:32] = 0.0                                   # a zero block
    w[5, :16] *= 1e-30                                  # a block near the bottom of f32
    w[7, 32:48] *= 1e30                                 # a block near the top
    p = orc.pack("nvfp8", w)
    s = p["scales"].view(np.float32).reshape(24, -1).astype(np.float64)
    codes = codes_of("nvfp8", p).reshape(24, -1, 16)
    t = torch_e4m3_table()
    blocks = w.astype(np.float64).reshape(24, -1, 16)
    amax = np.abs(blocks).max(-1)
    nz = amax > 0
    top = np.abs(blocks).argmax(-1)
    top_code = np.take_along_axis(codes, top[..., None], -1)[..., 0]
    assert ((top_code[nz] & 0x7F) == 0x7E).all(), np.argwhere(nz & ((top_code & 0x7F) != 0x7E))[:5]
    assert t[0x7E] == 448.0
    recon = t[top_code] * s
    top_val = np.take_along_axis(blocks, top[..., None], -1)[..., 0]
    assert (np.abs(recon[nz] - top_val[nz]) <= 2.0 ** -22 * amax[nz]).all()
    want = (amax.astype(np.float32) / np.float32(448.0)).astype(np.float64)
    assert (s[nz] == want[nz]).all()
    assert (s[~nz] == 1.0).all() and (codes[~nz] == 0).all()


def test_nonfinite_rejected(orc):
    w = np.zeros((2, 32), dtype=np.float32)
    w[1, 3] = np.nan
    with pytest.raises(orc.OracleError):
        orc.pack("mxfp4", w)
    w[1, 3] = np.inf
    with pytest.raises(orc.OracleError):
        orc.pack("int8_sym", w)


# ---------------------------------------------------------------- dequant
def _dequant_reference(fmt, p):
    c = codes_of(fmt, p)
    table = elem_table(fmt)
    with np.errstate(over="ignore", invalid="ignore"):
        S = np.repeat(scales_f64(fmt, p) / (np.float64(p["global"]) if fmt == "nvfp4" else 1.0), BLOCK[fmt], axis=1)
        v = table[c] * S
        if fmt == "nvfp4":
            v = v * np.float64(p["global"])
        if fmt == "int4_affine":
            v = v + np.repeat(bf16_to_f64(p["biases"].view(np.uint16)).reshape(p["n"], -1), 64, axis=1)
        return v.astype(np.float32)


def _same_f32(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    nan = np.isnan(a) & np.isnan(b)
    return ((a.view(np.uint32) == b.view(np.uint32)) | nan).all()


@pytest.mark.parametrize("fmt", ALL)
def test_dequant_matches_table_decode(orc, fmt):
    w = workloads.random_weights(16, 512, seed=1000, sigma=1.0, outliers=True)
    p = orc.pack(fmt, w)
    assert _same_f32(orc.dequant_packed(p), _dequant_reference(fmt, p))


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8_e4m3", "mxfp8_e5m2"])
def test_dequant_exhaustive_codes_times_all_e8m0(orc, fmt):
    ncode = 16 if fmt == "mxfp4" else 256
    n, k = 256, 256 if fmt == "mxfp4" else 8192  # row = one scale byte, all codes
    codes = np.tile(np.arange(ncode), (n, k // ncode))
    if fmt == "mxfp4":
        raw = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8).reshape(-1)
    else:
        raw = codes.astype(np.uint8).reshape(-1)
    scales = np.repeat(np.arange(256, dtype=np.uint8), k // 32)
    p = {"fmt": orc.FORMATS[fmt], "n": n, "k": k, "codes": raw, "scales": scales, "biases": None, "global": 1.0}
    got = orc.dequant_packed(p)
    assert _same_f32(got, _dequant_reference(fmt, p))
    # -0 stays -0 for finite scales
    neg0 = 8 if fmt == "mxfp4" else 0x80
    assert np.signbit(got[:255, neg0]).all()


def test_dequant_nvfp4_all_micro_codes(orc):
    n, k = 256, 16 * 16
    codes = np.tile(np.arange(16), (n, k // 16))
    raw = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8).reshape(-1)
    scales = np.repeat(np.arange(256, dtype=np.uint8), k // 16)
    for g in [1.0, 7.44e-6, 0.0014506777, 3.0e30]:
        p = {"fmt": orc.NVFP4, "n": n, "k": k, "codes": raw, "scales": scales, "biases": None,
             "global": float(np.float32(g))}
        assert _same_f32(orc.dequant_packed(p), _dequant_reference("nvfp4", p))


def test_dequant_int_formats_sweep(orc):
    rng = np.random.default_rng(5)
    n, k = 64, 256
    raw8 = np.tile(np.arange(256, dtype=np.uint8), n * k // 256)
    s32 = (rng.standard_normal(n * k // 32) * 1e-2).astype(np.float32)
    p = {"fmt": orc.INT8_SYM, "n": n, "k": k, "codes": raw8, "scales": s32.view(np.uint8), "biases": None, "global": 1.0}
    assert _same_f32(orc.dequant_packed(p), _dequant_reference("int8_sym", p))
    raw4 = np.tile(np.arange(256, dtype=np.uint8), n * k // 2 // 256)
    sb = torch.from_numpy((rng.standard_normal(n * k // 64) * 1e-2).astype(np.float32)).to(torch.bfloat16)
    bb = torch.from_numpy((rng.standard_normal(n * k // 64) * 1e-1).astype(np.float32)).to(torch.bfloat16)
    p = {"fmt": orc.INT4_AFFINE, "n": n, "k": k, "codes": raw4, "scales": sb.view(torch.uint16).numpy().view(np.uint8),
         "biases": bb.view(torch.uint16).numpy().view(np.uint8), "global": 1.0}
    assert _same_f32(orc.dequant_packed(p), _dequant_reference("int4_affine", p))
    s16 = (rng.standard_normal(n * k // 16) * 1e-3).astype(np.float32)
    p = {"fmt": orc.NVFP8, "n": n, "k": k, "codes": raw8, "scales": s16.view(np.uint8), "biases": None, "global": 1.0}
    assert _same_f32(orc.dequant_packed(p), _dequant_reference("nvfp8", p))


# ---------------------------------------------------------------- matmul
def test_matmul_matches_numpy_fp64(orc):
    rng = np.random.default_rng(31)
    x = rng.standard_normal((7, 300)).astype(np.float32)
    wd = rng.standard_normal((13, 300)).astype(np.float32)
    ref, den = orc.matmul(x, wd)
    want = x.astype(np.float64) @ wd.astype(np.float64).T
    wden = np.abs(x.astype(np.float64)) @ np.abs(wd.astype(np.float64)).T
    assert np.allclose(ref, want, rtol=0, atol=1e-12 * wden.max())
    assert np.allclose(den, wden, rtol=1e-13, atol=0)
    # rows subset and thread split do not change any value
    r2, d2 = orc.matmul(x, wd, rows=[6, 0, 3], threads=3)
    assert (r2 == ref[[6, 0, 3]]).all() and (d2 == den[[6, 0, 3]]).all()


def test_matmul_triple_loop_bit_identical(orc):
    rng = np.random.default_rng(32)
    x = rng.standard_normal((2, 9)).astype(np.float32)
    wd = rng.standard_normal((3, 9)).astype(np.float32)
    ref, den = orc.matmul(x, wd, threads=1)
    for i in range(2):
        for j in range(3):
            acc = 0.0
            mag = 0.0
            for p in range(9):
                t = float(x[i, p]) * float(wd[j, p])
                acc += t
                mag += abs(t)
            assert ref[i, j] == acc and den[i, j] == mag


def test_int4_algebraic_split_identity(orc):
    """The int4 reference's deterministic pattern: packs ((i+bit)&0xF) << 4*bit,
    scales 0.1 + 0.001 i, biases 1e-4 i, x = 1 + 0.001 i at m=8, n=16, k=512
    (scales/biases stored as bf16 here).  Dequant-then-dot must equal
    s * sum(q*x) + b * sum(x) per group."""
    m, n, k = 8, 16, 512
    G = k // 64
    words = np.zeros(n * k // 8, dtype=np.uint32)
    for bit in range(8):
        words |= ((np.arange(n * k // 8, dtype=np.uint32) + bit) & 0xF) << (4 * bit)
    s = torch.tensor([0.1 + 0.001 * i for i in range(n * G)], dtype=torch.float32).to(torch.bfloat16)
    b = torch.tensor([1e-4 * i for i in range(n * G)], dtype=torch.float32).to(torch.bfloat16)
    x = np.array([1.0 + 0.001 * i for i in range(m * k)], dtype=np.float32).reshape(m, k)
    p = {"fmt": orc.INT4_AFFINE, "n": n, "k": k, "codes": words.view(np.uint8),
         "scales": s.view(torch.uint16).numpy().view(np.uint8), "biases": b.view(torch.uint16).numpy().view(np.uint8),
         "global": 1.0}
    wd = orc.dequant_packed(p)
    ref, _ = orc.matmul(x, wd)
    q = codes_of("int4_affine", p).astype(np.float64).reshape(n, G, 64)
    s64 = s.double().numpy().reshape(n, G)
    b64 = b.double().numpy().reshape(n, G)
    xg = x.astype(np.float64).reshape(m, G, 64)
    split = np.einsum("ng,mgp,ngp->mn", s64, xg, q) + np.einsum("ng,mgp->mn", b64, xg)
    assert np.allclose(ref, split, rtol=1e-12, atol=0)


def test_matmul_rejects_bad_rows(orc):
    x = np.zeros((2, 4), np.float32)
    with pytest.raises(orc.OracleError):
        orc.matmul(x, np.zeros((3, 4), np.float32), rows=[2])


@pytest.mark.parametrize("xfmt,wfmt", [("mxfp8_e4m3", "mxfp4"), ("mxfp4", "mxfp4"), ("mxfp8_e5m2", "mxfp8_e4m3")])
def test_scaled_matmul_block_factorization(orc, xfmt, wfmt):
    """Both operands MX-packed: the oracle's dequant-then-dot equals the
    per-block form acc += (a_scale * b_scale) * sum dec(a) * dec(b) of the
    pages' TN scaled matmul, computed here from independent decode tables."""
    m, n, k = 5, 7, 256
    X = workloads.random_activations(m, k, seed=3, act="f32")
    W = workloads.random_weights(n, k, seed=4, sigma=0.02, outliers=True)
    px, pw = orc.pack(xfmt, X), orc.pack(wfmt, W)
    ref, _ = orc.matmul(orc.dequant_packed(px), orc.dequant_packed(pw))
    ca, cb = codes_of(xfmt, px).reshape(m, k // 32, 32), codes_of(wfmt, pw).reshape(n, k // 32, 32)
    da, db = elem_table(xfmt)[ca], elem_table(wfmt)[cb]
    sa, sb = scales_f64(xfmt, px), scales_f64(wfmt, pw)  # [m, k/32], [n, k/32]
    blk = np.einsum("mbp,nbp->mnb", da, db)
    want = np.einsum("mnb,mb,nb->mn", blk, sa, sb)
    assert np.allclose(ref, want, rtol=1e-12, atol=1e-300)
