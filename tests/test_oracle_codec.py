"""Pins for the oracle's element codec (CPU only).

Each decoder is checked against something other than itself: the values the
pages print (tests/golden), IEEE binary16 (numpy), or torch's float8 dtypes.
Each encoder is checked by brute force: the chosen code must be a nearest
grid point, ties must go to the even mantissa, and out-of-range inputs must
saturate.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_pairs(name, hexcode=False):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()
            out.append((int(a, 16) if hexcode else int(a), float(b)))
    return out


# Independent decode tables (library routines, not the oracle).
def torch_e4m3_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def half_e5m2_table():
    return (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)


def torch_e8m0_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()


def golden_e2m1_table():
    mags = dict(_read_pairs("e2m1_codebook.txt"))
    t = np.array([mags[c & 7] for c in range(16)], dtype=np.float64)
    t[8:] *= -1.0
    return t


def test_e2m1_matches_printed_codebook(orc):
    for code, value in _read_pairs("e2m1_codebook.txt"):
        assert orc.e2m1_value(code) == value
        assert orc.e2m1_value(code | 8) == -value
    assert math.copysign(1.0, orc.e2m1_value(8)) == -1.0  # -0 keeps its sign


def test_e2m1_matches_torch_fp4_unpack(orc):
    # torch's float4_e2m1fn_x2 has no arithmetic, but it round-trips through
    # float32 conversions in recent versions; fall back to the golden table.
    table = golden_e2m1_table()
    for c in range(16):
        v = orc.e2m1_value(c)
        assert v == table[c] and math.copysign(1, v) == math.copysign(1, table[c])


def test_e4m3_golden_points(orc):
    for code, value in _read_pairs("e4m3_points.txt", hexcode=True):
        assert orc.e4m3_value(code) == value, hex(code)


def test_e4m3_all_codes_match_torch_float8_e4m3fn(orc):
    t = torch_e4m3_table()
    for c in range(256):
        v = orc.e4m3_value(c)
        if math.isnan(t[c]):
            assert math.isnan(v), hex(c)
        else:
            assert v == t[c] and math.copysign(1, v) == math.copysign(1, t[c]), hex(c)
    # exactly two NaN codes, no inf
    assert sum(math.isnan(orc.e4m3_value(c)) for c in range(256)) == 2
    assert not any(math.isinf(orc.e4m3_value(c)) for c in range(256))


def test_e5m2_all_codes_match_ieee_half_high_byte(orc):
    t = half_e5m2_table()
    for c in range(256):
        v = orc.e5m2_value(c)
        if math.isnan(t[c]):
            assert math.isnan(v), hex(c)
        else:
            assert v == t[c] and math.copysign(1, v) == math.copysign(1, t[c]), hex(c)
    assert orc.e5m2_value(0x7B) == 57344.0


def test_e8m0_golden_and_torch(orc):
    for b, value in _read_pairs("e8m0_points.txt"):
        assert orc.e8m0_value(b) == value
    t = torch_e8m0_table()
    for b in range(256):
        v = orc.e8m0_value(b)
        if math.isnan(t[b]):
            assert math.isnan(v)
        else:
            assert v == t[b] == math.ldexp(1.0, b - 127)
    assert math.isnan(orc.e8m0_value(255))


# ---------------------------------------------------------------- encoders
def _finite_codes(table):
    return [c for c in range(len(table)) if np.isfinite(table[c])]


def _brute_nearest(v, table, codes):
    """All codes at minimal distance to v (ignoring sign of zero)."""
    d = np.array([abs(table[c] - v) for c in codes])
    best = d.min()
    return [codes[i] for i in np.nonzero(d == best)[0]], best


def _probe_values(table, vmax, rng):
    mags = sorted(set(abs(x) for x in table if np.isfinite(x)))
    vals = list(mags)
    vals += [(a + b) / 2 for a, b in zip(mags[:-1], mags[1:])]  # midpoints (ties)
    vals += [np.nextafter((a + b) / 2, 0) for a, b in zip(mags[:-1], mags[1:])]
    vals += [np.nextafter((a + b) / 2, np.inf) for a, b in zip(mags[:-1], mags[1:])]
    vals += list(rng.uniform(0, vmax * 1.2, 400)) + list(np.exp(rng.uniform(-12, math.log(vmax), 400)))
    vals += [vmax * 1.01, vmax * 1.2, vmax * 4, 1e30]
    vals = vals + [-v for v in vals]
    return vals


@pytest.mark.parametrize("name", ["e2m1", "e4m3", "e5m2"])
def test_encoder_bruteforce_nearest_ties_even_saturating(orc, name):
    rng = np.random.default_rng(7)
    if name == "e2m1":
        table, enc, vmax, sign = golden_e2m1_table(), orc.e2m1_encode, 6.0, 8
    elif name == "e4m3":
        table, enc, vmax, sign = torch_e4m3_table(), orc.e4m3_encode, 448.0, 0x80
    else:
        table, enc, vmax, sign = half_e5m2_table(), orc.e5m2_encode, 57344.0, 0x80
    codes = _finite_codes(table)
    for v in _probe_values(table, vmax, rng):
        c = enc(v)
        assert c in codes, (v, c)
        if abs(v) >= vmax:
            assert abs(table[c]) == vmax, (v, c)
            continue
        near, _ = _brute_nearest(v, table, codes)
        assert table[c] in [table[x] for x in near], (v, c, near)
        mags = {abs(table[x]) for x in near}
        if len(mags) > 1:  # a genuine tie between two grid points: even mantissa
            assert (c & 1) == 0, (v, c, near)
        # sign bit follows the input
        assert bool(c & sign) == (v < 0 or (v == 0 and math.copysign(1, v) < 0)), (v, c)


def test_e4m3_encoder_matches_torch_cast_in_range(orc):
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.standard_normal(2000) * 50, rng.uniform(-448, 448, 2000),
                        np.exp(rng.uniform(-14, 6, 2000))]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for x, r in zip(v, ref):
        assert orc.e4m3_encode(float(x)) == r, x


def test_e5m2_encoder_matches_torch_cast_in_range(orc):
    rng = np.random.default_rng(12)
    v = np.concatenate([rng.standard_normal(2000) * 1000, rng.uniform(-57344, 57344, 2000),
                        np.exp(rng.uniform(-20, 10, 2000))]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e5m2).view(torch.uint8).numpy()
    for x, r in zip(v, ref):
        assert orc.e5m2_encode(float(x)) == r, x


def test_torch_cast_does_not_saturate_so_oracle_clamps(orc):
    # torch's cast maps 480 to NaN; the pages' encoder saturates to 448.
    t = torch.tensor([480.0]).to(torch.float8_e4m3fn).view(torch.uint8).item()
    assert t == 0x7F
    assert orc.e4m3_encode(480.0) == 0x7E


def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(13)
    v = np.concatenate([rng.standard_normal(5000), np.exp(rng.uniform(-80, 80, 5000)) * np.sign(rng.standard_normal(5000))])
    v = v.astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    for x, r in zip(v, ref):
        assert orc.bf16_bits(float(x)) == r, x
