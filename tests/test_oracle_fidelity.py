"""Per-format fidelity of pack -> dequant (the oracle's), judged by direction.

The pages test block quantization by the cosine between the original and the
round-tripped weight against a per-format floor (metaltile PR #250, body of
the format commit: pack-then-dequant cosine per format), rather than by the
worst element.  They print no floor values, so each floor here comes from the
format's resolution with a margin:

* a float element with b mantissa bits rounds a value v in [2^e, 2^(e+1))
  to within half an ulp, ulp = 2^(e-b), so the relative error is uniform
  within at most +-2^-(b+1) and its RMS is at most 2^-(b+1)/sqrt(3); then
  cos = 1 - rel^2/2 >= 1 - 2^-2b/24: E4M3 (b=3) 0.99935 -> floor 0.999;
  E5M2 (b=2) 0.9974 -> floor 0.997; E2M1 (b=1) 0.9896 -> floor 0.985, the
  margin for the block's small values that fall below E2M1's 0.5 subnormal
  and round to zero;
* int4 affine: 15 steps over a 64-group's range (about 4.8 sigma for a
  Gaussian), RMS error step/sqrt(12) ~ 0.093 sigma -> cos ~ 0.9957, floor
  0.994; with 1% outliers at 50x a group's range is the outlier's, floor 0.98;
* int8 symmetric: 127 steps over a 32-block's amax (~2.1 sigma), RMS error
  ~0.005 sigma -> floor 0.9999 (0.9998 with outliers).

The same floors hold for the matmul outputs against the unquantized product
(X drawn independently of W, so the output error is the weight error seen
through X).  Measured values (seed below, 512 x 4096):

    format       N(0,.02): cos   rel.err   with 1% x50 outliers: cos   rel.err
    mxfp4        0.99350  0.1140     0.98964  0.1499
    nvfp4        0.99548  0.0951     0.99789  0.0649
    mxfp8_e4m3   0.99957  0.0293     0.99926  0.0395
    mxfp8_e5m2   0.99855  0.0538     0.99836  0.0584
    nvfp8        0.99975  0.0223     0.99998  0.0061
    int4_affine  0.99602  0.0895     0.98530  0.1739
    int8_sym     0.99999  0.0053     0.99993  0.0121
"""
import numpy as np
import pytest

import oracle
from block_scaled_bit_e2m1_amd import workloads

FLOOR = {  # (Gaussian weights, with outliers)
    "mxfp4": (0.985, 0.985),
    "nvfp4": (0.985, 0.985),
    "mxfp8_e4m3": (0.999, 0.999),
    "mxfp8_e5m2": (0.997, 0.997),
    "nvfp8": (0.999, 0.999),
    "int4_affine": (0.994, 0.98),
    "int8_sym": (0.9999, 0.9998),
}


def _cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / np.sqrt((a @ a) * (b @ b)))


@pytest.fixture(scope="module")
def data():
    return (workloads.random_weights(512, 4096, seed=5, sigma=0.02, outliers=False),
            workloads.random_weights(512, 4096, seed=6, sigma=0.02, outliers=True),
            workloads.random_activations(16, 4096, seed=7, act="bf16"))


@pytest.mark.parametrize("fmt", list(FLOOR))
def test_pack_dequant_cosine_floor(fmt, data):
    W, Wo, X = data
    for w, floor, what in ((W, FLOOR[fmt][0], "gaussian"), (Wo, FLOOR[fmt][1], "outliers")):
        d = oracle.dequant_packed(oracle.pack(fmt, w))
        c = _cos(d, w)
        assert c >= floor, f"{fmt} {what}: weight cosine {c:.6f} < {floor}"
        y = X.astype(np.float64) @ w.astype(np.float64).T
        yq = X.astype(np.float64) @ d.astype(np.float64).T
        co = _cos(yq, y)
        assert co >= floor, f"{fmt} {what}: output cosine {co:.6f} < {floor}"
        assert c < 1.0  # a lossy format that reproduces its input exactly has not quantized it


def test_finer_formats_are_closer(data):
    """The ordering the element widths imply: 8-bit floats beat 4-bit floats,
    E4M3 (3 mantissa bits) beats E5M2 (2), and the 16-block formats beat
    their 32-block counterparts on Gaussian weights."""
    W = data[0]
    c = {f: _cos(oracle.dequant_packed(oracle.pack(f, W)), W) for f in FLOOR}
    assert c["mxfp8_e4m3"] > c["mxfp8_e5m2"] > c["nvfp4"] > c["mxfp4"]
    assert c["int8_sym"] > c["nvfp8"] > c["mxfp8_e4m3"]
    assert c["nvfp8"] > c["mxfp8_e4m3"] and c["nvfp4"] > c["mxfp4"]
