"""Plain CPU oracle for block-scaled dequantize-and-multiply (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it.

The arithmetic lives in ``oracle.c`` (plain C, fp64); this module only moves
numpy arrays in and out.  Build it with :func:`build` (gcc, no HIP).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

MXFP4, NVFP4, MXFP8_E4M3, MXFP8_E5M2, NVFP8, INT4_AFFINE, INT8_SYM = 1, 2, 3, 4, 5, 6, 7
FORMATS = {
    "mxfp4": MXFP4,
    "nvfp4": NVFP4,
    "mxfp8_e4m3": MXFP8_E4M3,
    "mxfp8_e5m2": MXFP8_E5M2,
    "nvfp8": NVFP8,
    "int4_affine": INT4_AFFINE,
    "int8_sym": INT8_SYM,
}

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def build() -> str:
    """Compile liboracle.so with gcc (-O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
           _SRC, "-o", _LIB, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        for name in ("orc_e2m1_value", "orc_e4m3_value", "orc_e5m2_value", "orc_e8m0_value"):
            getattr(L, name).restype = ctypes.c_double
            getattr(L, name).argtypes = [ctypes.c_uint]
        for name in ("orc_e2m1_encode", "orc_e4m3_encode", "orc_e5m2_encode"):
            getattr(L, name).restype = ctypes.c_uint
            getattr(L, name).argtypes = [ctypes.c_double]
        L.orc_bf16_bits.restype = ctypes.c_uint16
        L.orc_bf16_bits.argtypes = [ctypes.c_double]
        L.orc_block.restype = ctypes.c_int
        L.orc_block.argtypes = [ctypes.c_int]
        L.orc_sizes.restype = ctypes.c_int
        L.orc_sizes.argtypes = [ctypes.c_int, _i64, _i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64),
                                ctypes.POINTER(_i64)]
        L.orc_pack.restype = ctypes.c_int
        L.orc_pack.argtypes = [ctypes.c_int, _vp, _i64, _i64, _vp, _vp, _vp, ctypes.POINTER(ctypes.c_float)]
        L.orc_dequant.restype = ctypes.c_int
        L.orc_dequant.argtypes = [ctypes.c_int, _i64, _i64, _vp, _vp, _vp, ctypes.c_float, _vp]
        L.orc_matmul.restype = ctypes.c_int
        L.orc_matmul.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp, ctypes.c_int]
        L.orc_matmul_f64.restype = ctypes.c_int
        L.orc_matmul_f64.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp, ctypes.c_int]
        L.orc_gather_matmul.restype = ctypes.c_int
        L.orc_gather_matmul.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp]
        L.orc_rmsnorm.restype = ctypes.c_int
        L.orc_rmsnorm.argtypes = [_vp, _vp, _i64, _i64, ctypes.c_double, _vp]
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_vp)


# -- codec ----------------------------------------------------------------
def e2m1_value(c: int) -> float:
    return lib().orc_e2m1_value(c)


def e4m3_value(c: int) -> float:
    return lib().orc_e4m3_value(c)


def e5m2_value(c: int) -> float:
    return lib().orc_e5m2_value(c)


def e8m0_value(b: int) -> float:
    return lib().orc_e8m0_value(b)


def e2m1_encode(v: float) -> int:
    return lib().orc_e2m1_encode(float(v))


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(float(v))


def e5m2_encode(v: float) -> int:
    return lib().orc_e5m2_encode(float(v))


def bf16_bits(v: float) -> int:
    return lib().orc_bf16_bits(float(v))


def block(fmt) -> int:
    return lib().orc_block(_fmt(fmt))


def sizes(fmt, n: int, k: int):
    c, s, b = _i64(), _i64(), _i64()
    st = lib().orc_sizes(_fmt(fmt), n, k, ctypes.byref(c), ctypes.byref(s), ctypes.byref(b))
    if st:
        raise OracleError(f"orc_sizes status {st}")
    return c.value, s.value, b.value


_SCALE_DT = {MXFP4: np.uint8, NVFP4: np.uint8, MXFP8_E4M3: np.uint8, MXFP8_E5M2: np.uint8,
             NVFP8: np.float32, INT8_SYM: np.float32, INT4_AFFINE: np.uint16}


def pack(fmt, w: np.ndarray):
    """f32 [n,k] -> dict(codes, scales, biases, global). Codes are raw bytes
    (uint8 view of the u32 words for 4-bit formats)."""
    f = _fmt(fmt)
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    cb, sb, bb = sizes(f, n, k)
    codes = np.zeros(cb, dtype=np.uint8)
    scales = np.zeros(sb, dtype=np.uint8)
    biases = np.zeros(bb, dtype=np.uint8) if bb else None
    g = ctypes.c_float(0.0)
    st = lib().orc_pack(f, _ptr(w), n, k, _ptr(codes), _ptr(scales), _ptr(biases), ctypes.byref(g))
    if st:
        raise OracleError(f"orc_pack status {st}")
    return {"codes": codes, "scales": scales, "biases": biases, "global": float(g.value),
            "n": n, "k": k, "fmt": f}


def dequant(fmt, n, k, codes, scales, biases=None, global_scale=1.0) -> np.ndarray:
    f = _fmt(fmt)
    out = np.empty((n, k), dtype=np.float32)
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    biases = None if biases is None else np.ascontiguousarray(biases)
    st = lib().orc_dequant(f, n, k, _ptr(codes), _ptr(scales), _ptr(biases), ctypes.c_float(global_scale),
                           _ptr(out))
    if st:
        raise OracleError(f"orc_dequant status {st}")
    return out


def dequant_packed(p: dict) -> np.ndarray:
    return dequant(p["fmt"], p["n"], p["k"], p["codes"], p["scales"], p["biases"], p["global"])


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """fp64 [m,k]: x * g / sqrt(mean(x^2) + eps) per row (f32 x and g values)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    g = np.ascontiguousarray(g, dtype=np.float32)
    m, k = x.shape
    if g.shape != (k,):
        raise OracleError("g must have k elements")
    out = np.empty((m, k), dtype=np.float64)
    st = lib().orc_rmsnorm(_ptr(x), _ptr(g), m, k, ctypes.c_double(eps), _ptr(out))
    if st:
        raise OracleError(f"orc_rmsnorm status {st}")
    return out


def gather_matmul(x: np.ndarray, wd_stack: np.ndarray, ids: np.ndarray, n: int):
    """ref, den (fp64 [m, n]): row i of X times expert ids[i] of the stack
    Wd [E*n, k] (rows ids[i]*n .. ids[i]*n + n - 1)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    wd_stack = np.ascontiguousarray(wd_stack, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    m, k = x.shape
    if wd_stack.shape[1] != k or wd_stack.shape[0] % n or ids.shape != (m,):
        raise OracleError("shape mismatch")
    E = wd_stack.shape[0] // n
    ref = np.empty((m, n), dtype=np.float64)
    den = np.empty((m, n), dtype=np.float64)
    st = lib().orc_gather_matmul(_ptr(x), _ptr(wd_stack), _ptr(ids), m, n, k, E, _ptr(ref), _ptr(den))
    if st:
        raise OracleError(f"orc_gather_matmul status {st}")
    return ref, den


def matmul(x: np.ndarray, wd: np.ndarray, rows=None, threads: int | None = None):
    """ref, den (fp64 [len(rows), n]) for rows of X times Wd^T.  X is taken as
    f32 values, or as fp64 when it is a float64 array (a normalized activation)."""
    f64 = x.dtype == np.float64
    x = np.ascontiguousarray(x, dtype=np.float64 if f64 else np.float32)
    wd = np.ascontiguousarray(wd, dtype=np.float32)
    m, k = x.shape
    n, k2 = wd.shape
    if k != k2:
        raise OracleError("k mismatch")
    if rows is None:
        r = None
        nr = m
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        nr = len(r)
    ref = np.empty((nr, n), dtype=np.float64)
    den = np.empty((nr, n), dtype=np.float64)
    if threads is None:
        threads = max(1, min(16, os.cpu_count() or 1))
    fn = lib().orc_matmul_f64 if f64 else lib().orc_matmul
    st = fn(_ptr(x), _ptr(wd), m, n, k, _ptr(r), nr, _ptr(ref), _ptr(den), threads)
    if st:
        raise OracleError(f"orc_matmul status {st}")
    return ref, den
