"""Python binding for libbsq.so (ctypes; argument marshalling only).

The functions named ``bsq_*`` mirror the C ABI in ``include/bsq.h`` one to one
and take raw pointers / sizes.  The helpers below them (``pack``, ``to_device``,
``dequant``, ``qgemv``, ``qgemm``) take torch tensors, pass their data
pointers and the current HIP stream, and raise :class:`BsqError` on a non-OK
status.  Every step of the computation runs in the library's HIP kernels (or
its C++ host packer); nothing here computes, and there is no fallback: if the
library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch  # loaded first so libbsq.so binds to the HIP runtime torch already holds

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbsq.so")

# bsq_format
MXFP4, NVFP4, MXFP8_E4M3, MXFP8_E5M2, NVFP8, INT4_AFFINE, INT8_SYM = 1, 2, 3, 4, 5, 6, 7
FORMATS = {"mxfp4": MXFP4, "nvfp4": NVFP4, "mxfp8_e4m3": MXFP8_E4M3, "mxfp8_e5m2": MXFP8_E5M2, "nvfp8": NVFP8,
           "int4_affine": INT4_AFFINE, "int8_sym": INT8_SYM}
# bsq_dtype
F32, BF16 = 0, 1
# bsq_path
PATH_AUTO, PATH_ROWS, PATH_MFMA = 0, 1, 2
# bsq_status
OK, ERR_ARG, ERR_UNSUPPORTED, ERR_SHAPE, ERR_ALIGN, ERR_NONFINITE, ERR_HIP = 0, 1, 2, 3, 4, 5, 6

EXPORTS = ["bsq_packed_bytes", "bsq_pack_host", "bsq_quantize", "bsq_dequant", "bsq_qgemv", "bsq_qgemm", "bsq_qgemm_path",
           "bsq_qgemm_mx", "bsq_rmsnorm_qgemv", "bsq_gather_qmm", "bsq_grouped_qgemm_workspace", "bsq_grouped_qgemm",
           "bsq_grouped_qgemm_noalloc", "bsq_calib_read", "bsq_calib_mfma",
           "bsq_status_string", "bsq_last_error", "bsq_version"]


class BsqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {bsq_status_string(status)} ({status}): {bsq_last_error()}")


_i64, _vp, _c_int, _f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
_sz = ctypes.POINTER(ctypes.c_size_t)
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with python -m block_scaled_bit_e2m1_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        L.bsq_packed_bytes.argtypes = [_c_int, _c_int, _i64, _i64, _sz, _sz, _sz]
        L.bsq_pack_host.argtypes = [_c_int, _c_int, _vp, _i64, _i64, _vp, _vp, _vp, ctypes.POINTER(_f32)]
        L.bsq_quantize.argtypes = [_c_int, _c_int, _vp, _c_int, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]
        L.bsq_qgemm_mx.argtypes = [_c_int, _vp, _vp, _c_int, _vp, _vp, _i64, _i64, _i64, _vp, _c_int, _vp]
        L.bsq_dequant.argtypes = [_c_int, _c_int, _i64, _i64, _vp, _vp, _vp, _f32, _vp, _vp]
        L.bsq_qgemv.argtypes = [_c_int, _c_int, _i64, _i64, _vp, _vp, _vp, _f32, _vp, _c_int, _vp, _c_int, _vp]
        L.bsq_qgemm.argtypes = [_c_int, _c_int, _i64, _i64, _i64, _vp, _vp, _vp, _f32, _vp, _c_int, _vp, _c_int, _vp]
        L.bsq_qgemm_path.argtypes = [_c_int] + L.bsq_qgemm.argtypes
        L.bsq_rmsnorm_qgemv.argtypes = [_c_int, _c_int, _i64, _i64, _i64, _vp, _vp, _vp, _f32, _vp, _vp, _f32, _c_int,
                                        _vp, _c_int, _vp]
        L.bsq_gather_qmm.argtypes = [_c_int, _c_int, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _f32, _vp, _vp, _c_int, _vp,
                                     _c_int, _vp, _vp]
        L.bsq_grouped_qgemm_workspace.argtypes = [_i64, _i64, _sz]
        L.bsq_grouped_qgemm.argtypes = [_c_int, _c_int, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _f32, _vp, _vp, _vp,
                                        _c_int, _vp, ctypes.c_size_t, _vp, _vp]
        L.bsq_grouped_qgemm_noalloc.argtypes = [_c_int, _c_int, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _f32, _vp, _vp,
                                                _vp, _c_int, _vp, _vp]
        L.bsq_calib_read.argtypes = [_vp, _i64, _vp, _vp]
        L.bsq_calib_mfma.argtypes = [_i64, _i64, _vp, _vp]
        for f in ("bsq_packed_bytes", "bsq_pack_host", "bsq_quantize", "bsq_dequant", "bsq_qgemv", "bsq_qgemm", "bsq_qgemm_path",
                  "bsq_qgemm_mx", "bsq_rmsnorm_qgemv", "bsq_gather_qmm", "bsq_grouped_qgemm_workspace",
                  "bsq_grouped_qgemm", "bsq_grouped_qgemm_noalloc", "bsq_calib_read", "bsq_calib_mfma"):
            getattr(L, f).restype = _c_int
        for f in ("bsq_status_string", "bsq_last_error", "bsq_version"):
            getattr(L, f).restype = ctypes.c_char_p
        L.bsq_status_string.argtypes = [_c_int]
        L.bsq_last_error.argtypes = []
        L.bsq_version.argtypes = []
        _lib = L
    return _lib


# --------------------------------------------------------------- raw C ABI
def bsq_packed_bytes(fmt, block, n, k):
    c, s, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    st = lib().bsq_packed_bytes(fmt, block, n, k, ctypes.byref(c), ctypes.byref(s), ctypes.byref(b))
    return st, c.value, s.value, b.value


def bsq_pack_host(fmt, block, w, n, k, codes, scales, biases, global_out):
    return lib().bsq_pack_host(fmt, block, w, n, k, codes, scales, biases, global_out)


def bsq_quantize(fmt, block, w, wt, n, k, codes, scales, biases, global_dev, status_dev, stream):
    return lib().bsq_quantize(fmt, block, w, wt, n, k, codes, scales, biases, global_dev, status_dev, stream)


def bsq_qgemm_mx(xfmt, x_codes, x_scales, wfmt, w_codes, w_scales, m, n, k, out, ot, stream):
    return lib().bsq_qgemm_mx(xfmt, x_codes, x_scales, wfmt, w_codes, w_scales, m, n, k, out, ot, stream)


def bsq_dequant(fmt, block, n, k, codes, scales, biases, global_scale, out, stream):
    return lib().bsq_dequant(fmt, block, n, k, codes, scales, biases, global_scale, out, stream)


def bsq_qgemv(fmt, block, n, k, codes, scales, biases, global_scale, x, xt, out, ot, stream):
    return lib().bsq_qgemv(fmt, block, n, k, codes, scales, biases, global_scale, x, xt, out, ot, stream)


def bsq_qgemm(fmt, block, m, n, k, codes, scales, biases, global_scale, x, xt, out, ot, stream):
    return lib().bsq_qgemm(fmt, block, m, n, k, codes, scales, biases, global_scale, x, xt, out, ot, stream)


def bsq_rmsnorm_qgemv(fmt, block, m, n, k, codes, scales, biases, global_scale, x, norm_weight, eps, xt, out, ot,
                      stream):
    return lib().bsq_rmsnorm_qgemv(fmt, block, m, n, k, codes, scales, biases, global_scale, x, norm_weight, eps, xt,
                                   out, ot, stream)


def bsq_gather_qmm(fmt, block, m, n, k, num_experts, codes, scales, biases, global_scale, expert_ids, x, xt, out, ot,
                   status_dev, stream):
    return lib().bsq_gather_qmm(fmt, block, m, n, k, num_experts, codes, scales, biases, global_scale, expert_ids, x,
                                xt, out, ot, status_dev, stream)


def bsq_grouped_qgemm_workspace(m, num_experts):
    n = ctypes.c_size_t(0)
    st = lib().bsq_grouped_qgemm_workspace(m, num_experts, ctypes.byref(n))
    return st, n.value


def bsq_grouped_qgemm(fmt, block, m, n, k, num_experts, codes, scales, biases, global_scale, expert_ids, x, out, ot,
                      workspace, workspace_bytes, status_dev, stream):
    return lib().bsq_grouped_qgemm(fmt, block, m, n, k, num_experts, codes, scales, biases, global_scale, expert_ids,
                                   x, out, ot, workspace, workspace_bytes, status_dev, stream)


def bsq_grouped_qgemm_noalloc(fmt, block, m, n, k, num_experts, codes, scales, biases, global_scale, expert_ids, x,
                              out, ot, status_dev, stream):
    return lib().bsq_grouped_qgemm_noalloc(fmt, block, m, n, k, num_experts, codes, scales, biases, global_scale,
                                           expert_ids, x, out, ot, status_dev, stream)


def bsq_calib_read(buf, nbytes, sink, stream):
    return lib().bsq_calib_read(buf, nbytes, sink, stream)


def bsq_calib_mfma(iters, workgroups, sink, stream):
    return lib().bsq_calib_mfma(iters, workgroups, sink, stream)


def bsq_qgemm_path(path, fmt, block, m, n, k, codes, scales, biases, global_scale, x, xt, out, ot, stream):
    return lib().bsq_qgemm_path(path, fmt, block, m, n, k, codes, scales, biases, global_scale, x, xt, out, ot,
                                stream)


def bsq_status_string(status: int) -> str:
    return lib().bsq_status_string(status).decode()


def bsq_last_error() -> str:
    return lib().bsq_last_error().decode()


def bsq_version() -> str:
    return lib().bsq_version().decode()


# --------------------------------------------------------------- torch helpers
def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _check(st: int, where: str):
    if st != OK:
        raise BsqError(st, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


@dataclass
class PackedWeight:
    """A packed [n,k] weight: codes/scales/biases as uint8 tensors (host or device)."""
    fmt: int
    n: int
    k: int
    codes: torch.Tensor
    scales: torch.Tensor
    biases: torch.Tensor | None
    global_scale: float

    def to(self, device) -> "PackedWeight":
        mv = lambda t: None if t is None else t.to(device)
        return PackedWeight(self.fmt, self.n, self.k, mv(self.codes), mv(self.scales), mv(self.biases),
                            self.global_scale)

    @property
    def weight_bytes(self) -> int:
        return self.codes.numel() + self.scales.numel() + (0 if self.biases is None else self.biases.numel())


def packed_bytes(fmt, n: int, k: int, block: int = 0):
    st, c, s, b = bsq_packed_bytes(_fmt(fmt), block, n, k)
    _check(st, "bsq_packed_bytes")
    return c, s, b


def pack(fmt, w, block: int = 0) -> PackedWeight:
    """Pack a host f32 [n,k] weight (numpy array or CPU tensor) with the library's host packer."""
    f = _fmt(fmt)
    if isinstance(w, torch.Tensor):
        w = w.detach().cpu().numpy()
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    cb, sb, bb = packed_bytes(f, n, k, block)
    codes = torch.zeros(max(cb, 16), dtype=torch.uint8)[:cb]
    scales = torch.zeros(sb, dtype=torch.uint8)
    biases = torch.zeros(bb, dtype=torch.uint8) if bb else None
    g = ctypes.c_float(0.0)
    st = bsq_pack_host(f, block, w.ctypes.data_as(ctypes.c_void_p), n, k, _ptr(codes), _ptr(scales), _ptr(biases),
                       ctypes.byref(g))
    _check(st, "bsq_pack_host")
    return PackedWeight(f, n, k, codes, scales, biases, float(g.value))


def quantize(fmt, w: torch.Tensor, block: int = 0, check_finite: bool = True) -> PackedWeight:
    """Pack a device f32 [n,k] weight on the GPU (bsq_quantize).  The nvfp4
    global scale is read back to the host (one synchronizing copy)."""
    f = _fmt(fmt)
    if w.dtype not in (torch.float32, torch.bfloat16) or not w.is_cuda or not w.is_contiguous():
        raise ValueError("w must be a contiguous float32 or bfloat16 CUDA tensor")
    n, k = w.shape
    cb, sb, bb = packed_bytes(f, n, k, block)
    dev = w.device
    codes = torch.empty(max(cb, 16), dtype=torch.uint8, device=dev)[:cb]
    scales = torch.empty(max(sb, 4), dtype=torch.uint8, device=dev)[:sb]
    biases = torch.empty(max(bb, 2), dtype=torch.uint8, device=dev)[:bb] if bb else None
    gdev = torch.ones(1, dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    st = bsq_quantize(f, block, _ptr(w), _DT[w.dtype], n, k, _ptr(codes), _ptr(scales), _ptr(biases), _ptr(gdev),
                      _ptr(status) if check_finite else None, _stream(dev))
    _check(st, "bsq_quantize")
    if check_finite and int(status.item()) != OK:
        raise BsqError(int(status.item()), "bsq_quantize (device)")
    return PackedWeight(f, n, k, codes, scales, biases, float(gdev.item()) if f == NVFP4 else 1.0)


def qgemm_mx(xq: PackedWeight, w: PackedWeight, out: torch.Tensor | None = None, out_dtype=torch.bfloat16):
    """out = dequant(xq) @ dequant(w)^T on the scaled matrix cores (bsq_qgemm_mx);
    xq is an MX-packed [m,k] activation (bsq_quantize), w an MX-packed [n,k] weight."""
    if xq.k != w.k:
        raise ValueError(f"k mismatch: activations {xq.k}, weight {w.k}")
    dev = w.codes.device
    if out is None:
        out = torch.empty((xq.n, w.n), dtype=out_dtype, device=dev)
    st = bsq_qgemm_mx(xq.fmt, _ptr(xq.codes), _ptr(xq.scales), w.fmt, _ptr(w.codes), _ptr(w.scales), xq.n, w.n, w.k,
                      _ptr(out), _DT[out.dtype], _stream(dev))
    _check(st, "bsq_qgemm_mx")
    return out


def to_device(pw: PackedWeight, device="cuda") -> PackedWeight:
    return pw.to(device)


def dequant(pw: PackedWeight, out: torch.Tensor | None = None) -> torch.Tensor:
    dev = pw.codes.device
    if out is None:
        out = torch.empty((pw.n, pw.k), dtype=torch.float32, device=dev)
    st = bsq_dequant(pw.fmt, 0, pw.n, pw.k, _ptr(pw.codes), _ptr(pw.scales), _ptr(pw.biases), pw.global_scale,
                     _ptr(out), _stream(dev))
    _check(st, "bsq_dequant")
    return out


_DT = {torch.float32: F32, torch.bfloat16: BF16}


def qgemv(pw: PackedWeight, x: torch.Tensor, out: torch.Tensor | None = None, out_dtype=None) -> torch.Tensor:
    dev = pw.codes.device
    if out is None:
        out = torch.empty((pw.n,), dtype=out_dtype or x.dtype, device=dev)
    st = bsq_qgemv(pw.fmt, 0, pw.n, pw.k, _ptr(pw.codes), _ptr(pw.scales), _ptr(pw.biases), pw.global_scale,
                   _ptr(x), _DT[x.dtype], _ptr(out), _DT[out.dtype], _stream(dev))
    _check(st, "bsq_qgemv")
    return out


def rmsnorm_qgemv(pw: PackedWeight, x: torch.Tensor, norm_weight: torch.Tensor, eps: float,
                  out: torch.Tensor | None = None, out_dtype=None) -> torch.Tensor:
    """out = rmsnorm(x, norm_weight, eps) @ dequant(pw)^T, fused (bsq_rmsnorm_qgemv);
    x is [k] or [m,k], norm_weight [k] of x's dtype."""
    dev = pw.codes.device
    x2 = x.reshape(-1, pw.k)
    if norm_weight.dtype != x.dtype or norm_weight.numel() != pw.k:
        raise ValueError("norm_weight must be [k] with x's dtype")
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (pw.n,), dtype=out_dtype or x.dtype, device=dev)
    st = bsq_rmsnorm_qgemv(pw.fmt, 0, x2.shape[0], pw.n, pw.k, _ptr(pw.codes), _ptr(pw.scales), _ptr(pw.biases),
                           pw.global_scale, _ptr(x2), _ptr(norm_weight), float(eps), _DT[x.dtype], _ptr(out),
                           _DT[out.dtype], _stream(dev))
    _check(st, "bsq_rmsnorm_qgemv")
    return out


def gather_qmm(stack: PackedWeight, num_experts: int, expert_ids: torch.Tensor, x: torch.Tensor,
               out: torch.Tensor | None = None, out_dtype=None, status: torch.Tensor | None = None) -> torch.Tensor:
    """out[i] = x[i] @ dequant(expert expert_ids[i])^T for an expert stack
    packed as one [num_experts*n, k] weight (bsq_gather_qmm)."""
    if stack.n % num_experts:
        raise ValueError("stack rows must be num_experts * n")
    n = stack.n // num_experts
    if expert_ids.dtype != torch.int32 or expert_ids.numel() != x.shape[0]:
        raise ValueError("expert_ids must be int32 with one id per x row")
    dev = stack.codes.device
    if out is None:
        out = torch.empty((x.shape[0], n), dtype=out_dtype or x.dtype, device=dev)
    st = bsq_gather_qmm(stack.fmt, 0, x.shape[0], n, stack.k, num_experts, _ptr(stack.codes), _ptr(stack.scales),
                        _ptr(stack.biases), stack.global_scale, _ptr(expert_ids), _ptr(x), _DT[x.dtype], _ptr(out),
                        _DT[out.dtype], _ptr(status), _stream(dev))
    _check(st, "bsq_gather_qmm")
    return out


def grouped_qmm(stack: PackedWeight, num_experts: int, expert_ids: torch.Tensor, x: torch.Tensor,
                out: torch.Tensor | None = None, out_dtype=None, status: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The routed gather's result with the rows grouped by expert on the
    device (bsq_grouped_qgemm): x bf16 [m, k], one int32 expert id per row,
    stack packed as one [num_experts*n, k] weight.  `workspace` (a uint8 device
    tensor of at least bsq_grouped_qgemm_workspace bytes) is allocated here
    when not given."""
    if stack.n % num_experts:
        raise ValueError("stack rows must be num_experts * n")
    n = stack.n // num_experts
    m = x.shape[0]
    if expert_ids.dtype != torch.int32 or expert_ids.numel() != m:
        raise ValueError("expert_ids must be int32 with one id per x row")
    if x.dtype != torch.bfloat16:
        raise ValueError("grouped_qmm takes bf16 activations")
    dev = stack.codes.device
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype or x.dtype, device=dev)
    st, need = bsq_grouped_qgemm_workspace(m, num_experts)
    _check(st, "bsq_grouped_qgemm_workspace")
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    st = bsq_grouped_qgemm(stack.fmt, 0, m, n, stack.k, num_experts, _ptr(stack.codes), _ptr(stack.scales),
                           _ptr(stack.biases), stack.global_scale, _ptr(expert_ids), _ptr(x), _ptr(out),
                           _DT[out.dtype], _ptr(workspace), workspace.numel(), _ptr(status), _stream(dev))
    _check(st, "bsq_grouped_qgemm")
    return out


def qgemm(pw: PackedWeight, x: torch.Tensor, out: torch.Tensor | None = None, out_dtype=None,
          path: int = PATH_AUTO) -> torch.Tensor:
    dev = pw.codes.device
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, pw.n), dtype=out_dtype or x.dtype, device=dev)
    st = bsq_qgemm_path(path, pw.fmt, 0, m, pw.n, pw.k, _ptr(pw.codes), _ptr(pw.scales), _ptr(pw.biases),
                        pw.global_scale, _ptr(x), _DT[x.dtype], _ptr(out), _DT[out.dtype], _stream(dev))
    _check(st, "bsq_qgemm")
    return out
