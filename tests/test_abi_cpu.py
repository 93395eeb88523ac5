"""Host-side checks of the C-ABI library (no GPU needed).

* libbsq.so loads and exports every function include/bsq.h declares;
* argument validation returns the documented status before any launch;
* the library's host packer (an independent C++ implementation) is
  byte-identical to the oracle's pack on every workload shape.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from block_scaled_bit_e2m1_amd import bsq, workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "bsq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsq_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_header_function():
    L = bsq.lib()
    names = header_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(bsq.EXPORTS)
    assert bsq.bsq_version().startswith("bsq")


def test_status_strings():
    for s in range(7):
        assert bsq.bsq_status_string(s)
    assert bsq.bsq_status_string(99) == "unknown status"


@pytest.mark.parametrize("fmt,n,k,want", [
    ("mxfp4", 16, 512, (4096, 256, 0)),
    ("nvfp4", 4096, 4096, (8 << 20, 1 << 20, 0)),
    ("mxfp8_e4m3", 14336, 4096, (56 << 20, 14336 * 128, 0)),
    ("int4_affine", 11008, 4096, (11008 * 2048, 11008 * 128, 11008 * 128)),
    ("int8_sym", 11008, 4096, (11008 * 4096, 11008 * 512, 0)),
    ("nvfp8", 8, 48, (384, 8 * 3 * 4, 0)),
])
def test_packed_bytes(fmt, n, k, want, orc):
    assert bsq.packed_bytes(fmt, n, k) == want
    assert orc.sizes(fmt, n, k) == want


def test_validation_errors():
    null = None
    st, *_ = bsq.bsq_packed_bytes(99, 0, 4, 32)
    assert st == bsq.ERR_UNSUPPORTED
    st, *_ = bsq.bsq_packed_bytes(bsq.MXFP4, 16, 4, 32)
    assert st == bsq.ERR_UNSUPPORTED  # wrong block
    st, *_ = bsq.bsq_packed_bytes(bsq.MXFP4, 0, 4, 48)
    assert st == bsq.ERR_SHAPE
    st, *_ = bsq.bsq_packed_bytes(bsq.NVFP4, 0, -1, 32)
    assert st == bsq.ERR_ARG
    # matmul argument checks happen before any device call
    p = ctypes.c_void_p(16)
    assert bsq.bsq_qgemm(bsq.MXFP4, 0, 2, 4, 48, p, p, null, 1.0, p, bsq.BF16, p, bsq.BF16, null) == bsq.ERR_SHAPE
    assert bsq.bsq_qgemm(bsq.MXFP4, 0, 2, 4, 64, p, p, null, 1.0, p, 7, p, bsq.BF16, null) == bsq.ERR_ARG
    assert bsq.bsq_qgemm(bsq.MXFP4, 0, 2, 4, 64, None, p, null, 1.0, p, bsq.BF16, p, bsq.BF16, null) == bsq.ERR_ARG
    assert bsq.bsq_qgemm(bsq.INT4_AFFINE, 0, 2, 4, 64, p, p, null, 1.0, p, bsq.BF16, p, bsq.BF16, null) == bsq.ERR_ARG
    mis = ctypes.c_void_p(8)
    assert bsq.bsq_qgemm(bsq.MXFP4, 0, 2, 4, 64, mis, p, null, 1.0, p, bsq.BF16, p, bsq.BF16, null) == bsq.ERR_ALIGN
    assert bsq.bsq_qgemm(bsq.MXFP4, 0, 2, 4, 64, p, p, null, 1.0, mis, bsq.BF16, p, bsq.BF16, null) == bsq.ERR_ALIGN
    assert bsq.bsq_qgemm(bsq.MXFP4, 0, 2, 4, 64, p, p, null, 1.0, p, bsq.BF16, ctypes.c_void_p(17), bsq.BF16,
                         null) == bsq.ERR_ALIGN
    assert bsq.bsq_qgemm_path(bsq.PATH_MFMA, bsq.MXFP4, 0, 2, 4, 64, p, p, null, 1.0, p, bsq.F32, p, bsq.F32,
                              null) == bsq.ERR_UNSUPPORTED
    assert bsq.bsq_qgemm_path(9, bsq.MXFP4, 0, 2, 4, 64, p, p, null, 1.0, p, bsq.BF16, p, bsq.BF16, null) == bsq.ERR_ARG
    assert bsq.bsq_dequant(bsq.MXFP4, 0, 4, 64, p, p, null, 1.0, ctypes.c_void_p(20), null) == bsq.ERR_ALIGN
    # empty shapes are accepted and launch nothing
    assert bsq.bsq_qgemm(bsq.MXFP4, 0, 0, 4, 64, None, None, null, 1.0, None, bsq.BF16, None, bsq.BF16, null) == bsq.OK
    assert bsq.bsq_qgemv(bsq.MXFP4, 0, 0, 64, None, None, null, 1.0, None, bsq.BF16, None, bsq.BF16, null) == bsq.OK
    assert bsq.bsq_dequant(bsq.MXFP4, 0, 0, 64, None, None, null, 1.0, None, null) == bsq.OK
    assert "aligned" in bsq.bsq_last_error() or bsq.bsq_last_error() == ""
    # calibration entry points: validation before any launch
    assert bsq.bsq_calib_read(p, 40, p, null) == bsq.ERR_SHAPE
    assert bsq.bsq_calib_read(p, -16, p, null) == bsq.ERR_ARG
    assert bsq.bsq_calib_read(mis, 64, p, null) == bsq.ERR_ALIGN
    assert bsq.bsq_calib_read(None, 64, p, null) == bsq.ERR_ARG
    assert bsq.bsq_calib_read(None, 0, None, null) == bsq.OK
    assert bsq.bsq_calib_mfma(10, 0, p, null) == bsq.ERR_ARG
    assert bsq.bsq_calib_mfma(-1, 4, p, null) == bsq.ERR_ARG
    assert bsq.bsq_calib_mfma(10, 4, None, null) == bsq.ERR_ARG


def test_pack_rejects_nonfinite():
    w = np.zeros((2, 32), np.float32)
    w[1, 1] = np.nan
    with pytest.raises(bsq.BsqError) as e:
        bsq.pack("mxfp4", w)
    assert e.value.status == bsq.ERR_NONFINITE


def _same_pack(p, q):
    return ((p["codes"] == q.codes.numpy()).all() and (p["scales"] == q.scales.numpy()).all()
            and (p["biases"] is None or (p["biases"] == q.biases.numpy()).all()) and p["global"] == q.global_scale)


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_library_pack_equals_oracle_pack(orc, name):
    wl = workloads.WORKLOADS[name]
    n = min(wl.n, 2048)  # full k, first rows of the workload's recipe
    W, _ = workloads.generate(wl, m=1, n=n)
    assert _same_pack(orc.pack(wl.fmt, W), bsq.pack(wl.fmt, W))


@pytest.mark.parametrize("fmt", list(bsq.FORMATS))
def test_library_pack_equals_oracle_pack_edge_values(orc, fmt):
    rng = np.random.default_rng(77)
    w = (rng.standard_normal((40, 256)) * np.exp(rng.uniform(-30, 30, (40, 1)))).astype(np.float32)
    w[0] = 0
    w[1, :64] = -0.0
    w[2] = np.float32(3.4e38) * np.sign(rng.standard_normal(256)).astype(np.float32)
    w[3] = np.float32(1e-45)
    w[4, ::2] = 6.0
    w[5] = np.linspace(-7, 7, 256, dtype=np.float32)
    assert _same_pack(orc.pack(fmt, w), bsq.pack(fmt, w))


def test_rmsnorm_qgemv_validation():
    """Argument checks of bsq_rmsnorm_qgemv happen before any launch."""
    import ctypes as C
    q = C.c_void_p(256)  # never dereferenced: every call below fails validation first
    f = bsq.bsq_rmsnorm_qgemv
    assert f(bsq.MXFP4, 0, 1, 4, 48, q, q, None, 1.0, q, q, 1e-6, bsq.BF16, q, bsq.BF16, None) == bsq.ERR_SHAPE  # k % 32
    assert f(bsq.MXFP4, 0, 1, 4, 64, q, q, None, 1.0, q, q, -1.0, bsq.BF16, q, bsq.BF16, None) == bsq.ERR_ARG  # eps < 0
    assert f(bsq.MXFP4, 0, 1, 4, 64, q, q, None, 1.0, q, q, float("nan"), bsq.BF16, q, bsq.BF16, None) == bsq.ERR_ARG
    assert f(bsq.MXFP4, 0, 1, 4, 64, q, q, None, 1.0, q, None, 1e-6, bsq.BF16, q, bsq.BF16, None) == bsq.ERR_ARG  # no g
    assert f(bsq.MXFP4, 0, 1, 4, 64, q, q, None, 1.0, q, C.c_void_p(258), 1e-6, bsq.BF16, q, bsq.BF16, None) == bsq.ERR_ALIGN
    assert f(bsq.MXFP4, 16, 1, 4, 64, q, q, None, 1.0, q, q, 1e-6, bsq.BF16, q, bsq.BF16, None) == bsq.ERR_UNSUPPORTED
    assert f(bsq.MXFP4, 0, 0, 4, 64, q, q, None, 1.0, q, q, 1e-6, bsq.BF16, q, bsq.BF16, None) == bsq.OK  # m = 0


def test_grouped_qgemm_workspace_and_validation():
    """bsq_grouped_qgemm_workspace's size (1 + 3 per possible 128-row tile +
    1 per row, in int32 words, the possible tiles being ceil(m/128) plus one
    per expert that can hold rows) and the grouped call's checks before any
    launch."""
    import ctypes as C
    W = bsq.bsq_grouped_qgemm_workspace
    assert W(2048, 8) == (bsq.OK, 4 * (1 + 3 * (16 + 8) + 2048))
    assert W(5, 1024) == (bsq.OK, 4 * (1 + 3 * (1 + 5) + 5))
    assert W(0, 4) == (bsq.OK, 4)
    assert W(10, 0)[0] == bsq.ERR_ARG and W(-1, 4)[0] == bsq.ERR_ARG
    assert W(10, 1025)[0] == bsq.ERR_SHAPE and W((1 << 24) + 1, 4)[0] == bsq.ERR_SHAPE
    q = C.c_void_p(256)  # never dereferenced: every call below returns before a launch
    f = bsq.bsq_grouped_qgemm
    ok_ws = 4 * (1 + 3 * (1 + 2) + 4)
    assert f(bsq.MXFP4, 0, 4, 64, 48, 2, q, q, None, 1.0, q, q, q, bsq.BF16, q, ok_ws, None, None) == bsq.ERR_SHAPE
    assert f(bsq.NVFP4, 0, 4, 64, 48, 2, q, q, None, 1.0, q, q, q, bsq.BF16, q, ok_ws, None, None) == bsq.ERR_SHAPE
    assert f(bsq.MXFP4, 0, 4, 64, 64, 0, q, q, None, 1.0, q, q, q, bsq.BF16, q, ok_ws, None, None) == bsq.ERR_ARG
    assert f(bsq.MXFP4, 0, 4, 64, 64, 1025, q, q, None, 1.0, q, q, q, bsq.BF16, q, ok_ws, None, None) == bsq.ERR_SHAPE
    assert f(bsq.MXFP4, 0, 4, 64, 64, 2, q, q, None, 1.0, q, q, q, 7, q, ok_ws, None, None) == bsq.ERR_ARG
    assert f(bsq.MXFP4, 0, 4, 64, 64, 2, q, q, None, 1.0, q, q, q, bsq.BF16, q, ok_ws - 4, None, None) == bsq.ERR_ARG
    assert f(bsq.MXFP4, 0, 4, 64, 64, 2, q, q, None, 1.0, q, q, q, bsq.BF16, None, ok_ws, None, None) == bsq.ERR_ARG
    assert f(bsq.MXFP4, 0, 4, 64, 64, 2, q, q, None, 1.0, None, q, q, bsq.BF16, q, ok_ws, None, None) == bsq.ERR_ARG
    assert f(bsq.MXFP4, 0, 4, 64, 64, 2, q, q, None, 1.0, q, C.c_void_p(264), q, bsq.BF16, q, ok_ws, None,
             None) == bsq.ERR_ALIGN
    assert f(bsq.MXFP4, 0, 4, 64, 64, 2, q, q, None, 1.0, q, q, q, bsq.BF16, C.c_void_p(258), ok_ws, None,
             None) == bsq.ERR_ALIGN
    assert f(bsq.INT4_AFFINE, 0, 4, 64, 64, 2, q, q, None, 1.0, q, q, q, bsq.BF16, q, ok_ws, None, None) == bsq.ERR_ARG
    assert f(bsq.MXFP4, 16, 4, 64, 64, 2, q, q, None, 1.0, q, q, q, bsq.BF16, q, ok_ws, None, None) == bsq.ERR_UNSUPPORTED
    assert f(bsq.MXFP4, 0, 0, 64, 64, 2, q, q, None, 1.0, q, q, q, bsq.BF16, None, 0, None, None) == bsq.OK  # m = 0
    assert f(bsq.MXFP4, 0, (1 << 24) + 1, 64, 64, 2, q, q, None, 1.0, q, q, q, bsq.BF16, q, ok_ws, None,
             None) == bsq.ERR_SHAPE


def test_bench_refuses_more_than_one_gpu():
    """The benchmark is one GPU's path: --gpus N > 1 exits with a message, before touching a device."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
