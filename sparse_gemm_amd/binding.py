"""Python face of the C ABI: a Pattern handle and the three compute calls on torch tensors.

PyTorch supplies device memory and the current stream; the arithmetic runs in the
library's HIP kernels. Names follow include/bsr_linear.h.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np
import torch  # imported before the library so the process maps a single HIP runtime

from . import _lib


def _single_hip_runtime() -> None:
    """Refuse to run with two different libamdhip64 images mapped (two HIP runtimes)."""
    try:
        with open("/proc/self/maps") as f:
            paths = {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    except OSError:
        return
    import os
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise RuntimeError(f"two HIP runtimes are mapped in this process: {sorted(real)}")


_checked = None
_hip_rt = None


def _hip() -> ctypes.CDLL:
    """The HIP runtime this process already maps (the one torch and the library share)."""
    global _hip_rt
    if _hip_rt is None:
        lib()
        with open("/proc/self/maps") as f:
            paths = sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
        if not paths:
            raise RuntimeError("no HIP runtime mapped")
        _hip_rt = ctypes.CDLL(paths[0])
    return _hip_rt


def device_int(addr: int) -> int:
    """The int32 at a device address (for example a device-built pattern's live nnzb), copied to
    the host after the device has finished its queued work."""
    torch.cuda.synchronize()
    v = ctypes.c_int32()
    rc = _hip().hipMemcpy(ctypes.byref(v), ctypes.c_void_p(addr), ctypes.c_size_t(4), 2)   # device to host
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed ({rc})")
    return v.value


def lib() -> ctypes.CDLL:
    global _checked
    if _checked is None:
        L = _lib.load()
        _single_hip_runtime()
        _checked = L
    return _checked


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


class Pattern:
    """A block pattern owned by the library: CSR, transposed CSC + perm, and work lists.

    Created from a block mask [N/b, K/b] (nonzero = kept block) or from CSR arrays. With
    upload=True (default) the metadata is copied to the current device; with False the
    pattern is host-only (export / info only)."""

    def __init__(self, handle: ctypes.c_void_p, upload: bool, device: Optional[int]):
        self._h = handle
        self.uploaded = upload
        self.device = device
        N, K, b, nnzb = (ctypes.c_int32() for _ in range(4))
        _lib.check(lib().bsr_pattern_info(self._h, ctypes.byref(N), ctypes.byref(K), ctypes.byref(b),
                                          ctypes.byref(nnzb)), "bsr_pattern_info")
        self.N, self.K, self.b, self.nnzb = N.value, K.value, b.value, nnzb.value
        self.R, self.C = self.N // self.b, self.K // self.b

    @staticmethod
    def _device(upload: bool) -> Optional[int]:
        if not upload:
            return None
        if not torch.cuda.is_available():
            raise RuntimeError("uploading a pattern needs a GPU")
        torch.cuda.init()
        return torch.cuda.current_device()

    @classmethod
    def from_mask(cls, mask, N: int, K: int, b: int, upload: bool = True) -> "Pattern":
        m = np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
        if m.shape != (N // b, K // b) or N % b or K % b:
            raise ValueError(f"mask shape {m.shape} does not match N={N}, K={K}, b={b}")
        dev = cls._device(upload)
        h = ctypes.c_void_p()
        _lib.check(lib().bsr_pattern_create_from_mask(N, K, b, m.ctypes.data_as(ctypes.c_void_p), int(upload),
                                                      ctypes.byref(h)), "bsr_pattern_create_from_mask")
        return cls(h, upload, dev)

    @classmethod
    def from_dense(cls, W: torch.Tensor, b: int, keep: int, kind: int = 1) -> "Pattern":
        """Pattern of the `keep` blocks of largest norm of the dense device weight W [N, K]
        (kind 1 = L1, 2 = squared L2), via bsr_pattern_create_from_dense."""
        N, K = W.shape
        dev = cls._device(True)
        _check_tensor(W, "W", (N, K), dev)
        h = ctypes.c_void_p()
        _lib.check(lib().bsr_pattern_create_from_dense(N, K, b, _ptr(W), int(kind), int(keep), _stream(dev),
                                                       ctypes.byref(h)), "bsr_pattern_create_from_dense")
        return cls(h, True, dev)

    @classmethod
    def from_csr(cls, N: int, K: int, b: int, row_ptr, col_idx, upload: bool = True) -> "Pattern":
        rp, ci = _i32(row_ptr), _i32(col_idx)
        dev = cls._device(upload)
        h = ctypes.c_void_p()
        _lib.check(lib().bsr_pattern_create_from_csr(N, K, b, int(ci.size), rp.ctypes.data_as(ctypes.c_void_p),
                                                     ci.ctypes.data_as(ctypes.c_void_p) if ci.size else None,
                                                     int(upload), ctypes.byref(h)), "bsr_pattern_create_from_csr")
        return cls(h, upload, dev)

    @classmethod
    def device_built(cls, N: int, K: int, b: int, cap: int) -> "Pattern":
        """An empty pattern whose metadata and work lists live on the device, rebuilt there from a
        device mask by rebuild() (bsr_pattern_create_device); nnzb reports the capacity cap."""
        dev = cls._device(True)
        h = ctypes.c_void_p()
        _lib.check(lib().bsr_pattern_create_device(N, K, b, int(cap), ctypes.byref(h)), "bsr_pattern_create_device")
        pat = cls(h, True, dev)
        pat.cap = int(cap)
        return pat

    def rebuild(self, mask: torch.Tensor) -> None:
        """Rebuild a device-built pattern from the device uint8 mask [N/b, K/b] on the current stream
        (bsr_pattern_rebuild; no host synchronisation)."""
        if mask.dtype != torch.uint8 or not mask.is_cuda or mask.device.index != self.device:
            raise ValueError(f"mask must be a uint8 tensor on cuda:{self.device}")
        if tuple(mask.shape) != (self.R, self.C) or not mask.is_contiguous():
            raise ValueError(f"mask must be a contiguous [{self.R}, {self.C}] tensor")
        _lib.check(lib().bsr_pattern_rebuild(self._h, _ptr(mask), _stream(self.device)), "bsr_pattern_rebuild")

    def device_arrays(self) -> dict:
        """Device addresses of a device-built pattern's row_ptr, col_idx, col_ptr, row_idx, perm and
        live nnzb (bsr_pattern_device_arrays)."""
        ptrs = [ctypes.c_void_p() for _ in range(6)]
        _lib.check(lib().bsr_pattern_device_arrays(self._h, *(ctypes.byref(q) for q in ptrs)),
                   "bsr_pattern_device_arrays")
        return dict(zip(("row_ptr", "col_idx", "col_ptr", "row_idx", "perm", "nnzb"), (q.value for q in ptrs)))

    def export(self) -> dict:
        out = dict(row_ptr=np.empty(self.R + 1, np.int32), col_idx=np.empty(self.nnzb, np.int32),
                   col_ptr=np.empty(self.C + 1, np.int32), row_idx=np.empty(self.nnzb, np.int32),
                   perm=np.empty(self.nnzb, np.int32))
        p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
        _lib.check(lib().bsr_pattern_export(self._h, p(out["row_ptr"]), p(out["col_idx"]), p(out["col_ptr"]),
                                            p(out["row_idx"]), p(out["perm"])), "bsr_pattern_export")
        return out

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    def close(self) -> None:
        if self._h is not None and self._h.value:
            if self.uploaded and torch.cuda.is_available():
                torch.cuda.synchronize(self.device)  # no queued kernel may still read the metadata
            _lib.load().bsr_pattern_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _check_tensor(t: torch.Tensor, name: str, shape, device) -> None:
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda or t.device.index != device:
        raise ValueError(f"{name} must be on cuda:{device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device: int):
    return torch.cuda.current_stream(device).cuda_stream


def linear_fwd(p: Pattern, X: torch.Tensor, V: torch.Tensor, bias: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X . W~^T + bias via bsr_linear_fwd; X [M, K], V [nnzb, b, b], bias [N] or None."""
    M = X.shape[0]
    _check_tensor(X, "X", (M, p.K), p.device)
    _check_tensor(V, "V", (p.nnzb, p.b, p.b), p.device)
    if bias is not None:
        _check_tensor(bias, "bias", (p.N,), p.device)
    if out is None:
        out = torch.empty((M, p.N), dtype=torch.bfloat16, device=X.device)
    _check_tensor(out, "out", (M, p.N), p.device)
    _lib.check(lib().bsr_linear_fwd(p.handle, _ptr(X), M, _ptr(V), _ptr(bias), _ptr(out), _stream(p.device)),
               "bsr_linear_fwd")
    return out


def linear_bwd_input(p: Pattern, dY: torch.Tensor, V: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dX = dY . W~ via bsr_linear_bwd_input; dY [M, N]."""
    M = dY.shape[0]
    _check_tensor(dY, "dY", (M, p.N), p.device)
    _check_tensor(V, "V", (p.nnzb, p.b, p.b), p.device)
    if out is None:
        out = torch.empty((M, p.K), dtype=torch.bfloat16, device=dY.device)
    _check_tensor(out, "out", (M, p.K), p.device)
    _lib.check(lib().bsr_linear_bwd_input(p.handle, _ptr(dY), M, _ptr(V), _ptr(out), _stream(p.device)),
               "bsr_linear_bwd_input")
    return out


def bwd_weight_workspace_bytes(p: Pattern, M: int) -> int:
    return int(lib().bsr_linear_bwd_weight_workspace(p.handle, int(M)))


def op_kernels(p: Pattern, op: str, M: int) -> list:
    """Names of the main kernels one call of op ("fwd", "dx", "dw" or "fwd_24") launches for M rows
    (the bias gradient's excluded), as the library dispatches them."""
    code = {"fwd": 0, "dx": 1, "dw": 2, "fwd_24": 3}[op]
    buf = ctypes.create_string_buffer(256)
    _lib.check(lib().bsr_op_kernels(p.handle, code, int(M), buf, len(buf)), "bsr_op_kernels")
    names = buf.value.decode()
    return names.split(",") if names else []


def linear_bwd_weight(p: Pattern, dY: torch.Tensor, X: torch.Tensor, want_dbias: bool = False,
                      out: Optional[torch.Tensor] = None, dbias: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None):
    """(dV, dbias or None) via bsr_linear_bwd_weight; dV [nnzb, b, b] on the pattern only."""
    M = dY.shape[0]
    _check_tensor(dY, "dY", (M, p.N), p.device)
    _check_tensor(X, "X", (M, p.K), p.device)
    if out is None:
        out = torch.empty((p.nnzb, p.b, p.b), dtype=torch.bfloat16, device=dY.device)
    _check_tensor(out, "out", (p.nnzb, p.b, p.b), p.device)
    if want_dbias and dbias is None:
        dbias = torch.empty((p.N,), dtype=torch.bfloat16, device=dY.device)
    if dbias is not None:
        _check_tensor(dbias, "dbias", (p.N,), p.device)
    need = bwd_weight_workspace_bytes(p, M)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dY.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _lib.check(lib().bsr_linear_bwd_weight(p.handle, _ptr(dY), _ptr(X), M, _ptr(out), _ptr(dbias), _ptr(workspace),
                                           ws_bytes, _stream(p.device)), "bsr_linear_bwd_weight")
    return out, dbias


def linear_bwd_weight_noalloc(p: Pattern, dY: torch.Tensor, X: torch.Tensor, out: torch.Tensor,
                              dbias: Optional[torch.Tensor] = None):
    """dV (and dbias) into caller-provided outputs via bsr_linear_bwd_weight_noalloc: the library's
    per-GPU scratch array instead of a workspace; nothing is allocated."""
    M = dY.shape[0]
    _check_tensor(dY, "dY", (M, p.N), p.device)
    _check_tensor(X, "X", (M, p.K), p.device)
    _check_tensor(out, "out", (p.nnzb, p.b, p.b), p.device)
    if dbias is not None:
        _check_tensor(dbias, "dbias", (p.N,), p.device)
    _lib.check(lib().bsr_linear_bwd_weight_noalloc(p.handle, _ptr(dY), _ptr(X), M, _ptr(out), _ptr(dbias),
                                                   _stream(p.device)), "bsr_linear_bwd_weight_noalloc")
    return out, dbias


# ---- dense <-> BSR conversion and block magnitudes (include/bsr_convert.h) ----

NORM_L1, NORM_L2_SQUARED = 1, 2


def block_norms(W: torch.Tensor, b: int, kind: int = NORM_L1, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp64 [N/b, K/b] block magnitudes of the dense device weight W [N, K] via bsr_block_norms."""
    N, K = W.shape
    dev = W.device.index
    _check_tensor(W, "W", (N, K), dev)
    if out is None:
        out = torch.empty((N // b, K // b), dtype=torch.float64, device=W.device)
    if out.dtype != torch.float64 or tuple(out.shape) != (N // b, K // b) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp64 [N/b, K/b] tensor")
    _lib.check(lib().bsr_block_norms(N, K, b, _ptr(W), int(kind), _ptr(out), _stream(dev)), "bsr_block_norms")
    return out


def mask_topk(norms, keep: int) -> np.ndarray:
    """Host [R, C] uint8 mask of the `keep` largest block norms (ties to the lower index)
    via bsr_mask_topk."""
    n = np.ascontiguousarray(np.asarray(norms, dtype=np.float64))
    R, C = n.shape
    mask = np.empty((R, C), dtype=np.uint8)
    _lib.check(lib().bsr_mask_topk(R, C, n.ctypes.data_as(ctypes.c_void_p), int(keep),
                                   mask.ctypes.data_as(ctypes.c_void_p)), "bsr_mask_topk")
    return mask


def dense_to_values(p: Pattern, W: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """V [nnzb, b, b]: the kept blocks of the dense device weight W [N, K], via bsr_dense_to_values."""
    _check_tensor(W, "W", (p.N, p.K), p.device)
    if out is None:
        out = torch.empty((p.nnzb, p.b, p.b), dtype=torch.bfloat16, device=W.device)
    _check_tensor(out, "out", (p.nnzb, p.b, p.b), p.device)
    _lib.check(lib().bsr_dense_to_values(p.handle, _ptr(W), _ptr(out), _stream(p.device)), "bsr_dense_to_values")
    return out


def values_to_dense(p: Pattern, V: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The dense [N, K] weight with zeros outside the kept blocks, via bsr_values_to_dense."""
    _check_tensor(V, "V", (p.nnzb, p.b, p.b), p.device)
    if out is None:
        out = torch.empty((p.N, p.K), dtype=torch.bfloat16, device=V.device)
    _check_tensor(out, "out", (p.N, p.K), p.device)
    _lib.check(lib().bsr_values_to_dense(p.handle, _ptr(V), _ptr(out), _stream(p.device)), "bsr_values_to_dense")
    return out


# ---- fp8 (OCP E4M3) block values with a power-of-two scale per block (include/bsr_fp8.h) ----

def values_quantize_fp8(p: Pattern, V: torch.Tensor, out=None):
    """(codes uint8 [nnzb, b, b], scale exponents int32 [nnzb]) via bsr_values_quantize_fp8."""
    _check_tensor(V, "V", (p.nnzb, p.b, p.b), p.device)
    if out is None:
        out = (torch.empty((p.nnzb, p.b, p.b), dtype=torch.uint8, device=V.device),
               torch.empty((p.nnzb,), dtype=torch.int32, device=V.device))
    V8, se = out
    _check_raw(V8, "V8", (p.nnzb, p.b, p.b), torch.uint8, p.device)
    _check_raw(se, "se", (p.nnzb,), torch.int32, p.device)
    _lib.check(lib().bsr_values_quantize_fp8(p.handle, _ptr(V), _ptr(V8), _ptr(se), _stream(p.device)),
               "bsr_values_quantize_fp8")
    return V8, se


def values_dequantize_fp8(p: Pattern, V8: torch.Tensor, se: torch.Tensor, out=None) -> torch.Tensor:
    """bf16 [nnzb, b, b] = code * 2^se via bsr_values_dequantize_fp8."""
    _check_raw(V8, "V8", (p.nnzb, p.b, p.b), torch.uint8, p.device)
    _check_raw(se, "se", (p.nnzb,), torch.int32, p.device)
    if out is None:
        out = torch.empty((p.nnzb, p.b, p.b), dtype=torch.bfloat16, device=V8.device)
    _check_tensor(out, "out", (p.nnzb, p.b, p.b), p.device)
    _lib.check(lib().bsr_values_dequantize_fp8(p.handle, _ptr(V8), _ptr(se), _ptr(out), _stream(p.device)),
               "bsr_values_dequantize_fp8")
    return out


def linear_fwd_fp8(p: Pattern, X: torch.Tensor, V8: torch.Tensor, se: torch.Tensor,
                   bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X . W8~^T + bias with fp8 block values, via bsr_linear_fwd_fp8."""
    M = X.shape[0]
    _check_tensor(X, "X", (M, p.K), p.device)
    _check_raw(V8, "V8", (p.nnzb, p.b, p.b), torch.uint8, p.device)
    _check_raw(se, "se", (p.nnzb,), torch.int32, p.device)
    if bias is not None:
        _check_tensor(bias, "bias", (p.N,), p.device)
    if out is None:
        out = torch.empty((M, p.N), dtype=torch.bfloat16, device=X.device)
    _check_tensor(out, "out", (M, p.N), p.device)
    _lib.check(lib().bsr_linear_fwd_fp8(p.handle, _ptr(X), M, _ptr(V8), _ptr(se), _ptr(bias), _ptr(out),
                                        _stream(p.device)), "bsr_linear_fwd_fp8")
    return out


def _check_raw(t: torch.Tensor, name: str, shape, dtype, device) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda or t.device.index != device:
        raise ValueError(f"{name} must be on cuda:{device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---- 2:4 sparsity inside each kept block (include/bsr_sparse24.h) ----

def values_compress_24(p: Pattern, V: torch.Tensor, out=None):
    """(Vc bf16 [nnzb, b, b/2], meta uint16-as-int16 [nnzb, b, b/16]) via bsr_values_compress_24."""
    _check_tensor(V, "V", (p.nnzb, p.b, p.b), p.device)
    if out is None:
        out = (torch.empty((p.nnzb, p.b, p.b // 2), dtype=torch.bfloat16, device=V.device),
               torch.empty((p.nnzb, p.b, p.b // 16), dtype=torch.int16, device=V.device))
    Vc, mt = out
    _check_tensor(Vc, "Vc", (p.nnzb, p.b, p.b // 2), p.device)
    _check_raw(mt, "meta", (p.nnzb, p.b, p.b // 16), torch.int16, p.device)
    _lib.check(lib().bsr_values_compress_24(p.handle, _ptr(V), _ptr(Vc), _ptr(mt), _stream(p.device)),
               "bsr_values_compress_24")
    return Vc, mt


def values_decompress_24(p: Pattern, Vc: torch.Tensor, mt: torch.Tensor, out=None) -> torch.Tensor:
    """Dense bf16 blocks [nnzb, b, b] via bsr_values_decompress_24."""
    _check_tensor(Vc, "Vc", (p.nnzb, p.b, p.b // 2), p.device)
    _check_raw(mt, "meta", (p.nnzb, p.b, p.b // 16), torch.int16, p.device)
    if out is None:
        out = torch.empty((p.nnzb, p.b, p.b), dtype=torch.bfloat16, device=Vc.device)
    _check_tensor(out, "out", (p.nnzb, p.b, p.b), p.device)
    _lib.check(lib().bsr_values_decompress_24(p.handle, _ptr(Vc), _ptr(mt), _ptr(out), _stream(p.device)),
               "bsr_values_decompress_24")
    return out


def linear_fwd_24(p: Pattern, X: torch.Tensor, Vc: torch.Tensor, mt: torch.Tensor,
                  bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X . W24~^T + bias with 2:4-compressed block values, via bsr_linear_fwd_24."""
    M = X.shape[0]
    _check_tensor(X, "X", (M, p.K), p.device)
    _check_tensor(Vc, "Vc", (p.nnzb, p.b, p.b // 2), p.device)
    _check_raw(mt, "meta", (p.nnzb, p.b, p.b // 16), torch.int16, p.device)
    if bias is not None:
        _check_tensor(bias, "bias", (p.N,), p.device)
    if out is None:
        out = torch.empty((M, p.N), dtype=torch.bfloat16, device=X.device)
    _check_tensor(out, "out", (M, p.N), p.device)
    _lib.check(lib().bsr_linear_fwd_24(p.handle, _ptr(X), M, _ptr(Vc), _ptr(mt), _ptr(bias), _ptr(out),
                                       _stream(p.device)), "bsr_linear_fwd_24")
    return out


# ---- on-device metadata rebuild (include/bsr_rebuild.h) ----

def meta_rebuild(mask: torch.Tensor, cap: Optional[int] = None) -> dict:
    """CSR / CSC / perm of a device block mask [R, C] (uint8) via bsr_meta_rebuild, asynchronous
    on the current stream. Returns device tensors row_ptr, col_idx, col_ptr, row_idx, perm (index
    arrays of length cap, default R*C) and nnzb (a 1-element device tensor)."""
    if mask.dtype != torch.uint8 or mask.dim() != 2 or not mask.is_cuda or not mask.is_contiguous():
        raise ValueError("mask must be a contiguous uint8 [R, C] device tensor")
    R, C = mask.shape
    cap = R * C if cap is None else int(cap)
    d = mask.device
    i32 = dict(dtype=torch.int32, device=d)
    out = dict(row_ptr=torch.empty(R + 1, **i32), col_idx=torch.empty(max(cap, 1), **i32),
               col_ptr=torch.empty(C + 1, **i32), row_idx=torch.empty(max(cap, 1), **i32),
               perm=torch.empty(max(cap, 1), **i32), nnzb=torch.empty(1, **i32))
    ws_bytes = int(lib().bsr_meta_rebuild_workspace(R, C))
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=d)
    _lib.check(lib().bsr_meta_rebuild(R, C, _ptr(mask), _ptr(out["row_ptr"]), _ptr(out["col_idx"]),
                                      _ptr(out["col_ptr"]), _ptr(out["row_idx"]), _ptr(out["perm"]), cap,
                                      _ptr(out["nnzb"]), _ptr(ws), ws_bytes,
                                      torch.cuda.current_stream(d).cuda_stream), "bsr_meta_rebuild")
    out["_workspace"] = ws   # keeps the scratch alive until the caller synchronises
    return out


def values_pack_24(p: Pattern, Vc: torch.Tensor, mt: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """2:4 block images [nnzb, b, b] (int16 units) for the large-M forward, via bsr_values_pack_24."""
    _check_tensor(Vc, "Vc", (p.nnzb, p.b, p.b // 2), p.device)
    _check_raw(mt, "meta", (p.nnzb, p.b, p.b // 16), torch.int16, p.device)
    if out is None:
        out = torch.empty((p.nnzb, p.b, p.b), dtype=torch.int16, device=Vc.device)
    _check_raw(out, "img", (p.nnzb, p.b, p.b), torch.int16, p.device)
    _lib.check(lib().bsr_values_pack_24(p.handle, _ptr(Vc), _ptr(mt), _ptr(out), _stream(p.device)),
               "bsr_values_pack_24")
    return out


def linear_fwd_24_image(p: Pattern, X: torch.Tensor, img: torch.Tensor, bias: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X . W24~^T + bias from 2:4 block images on the sparse matrix cores (any M), via
    bsr_linear_fwd_24_image."""
    M = X.shape[0]
    _check_tensor(X, "X", (M, p.K), p.device)
    _check_raw(img, "img", (p.nnzb, p.b, p.b), torch.int16, p.device)
    if bias is not None:
        _check_tensor(bias, "bias", (p.N,), p.device)
    if out is None:
        out = torch.empty((M, p.N), dtype=torch.bfloat16, device=X.device)
    _check_tensor(out, "out", (M, p.N), p.device)
    _lib.check(lib().bsr_linear_fwd_24_image(p.handle, _ptr(X), M, _ptr(img), _ptr(bias), _ptr(out),
                                             _stream(p.device)), "bsr_linear_fwd_24_image")
    return out


def values_quantize_fp8_24(p: Pattern, Vc: torch.Tensor, out=None):
    """(codes uint8 [nnzb, b, b/2], scale exponents int32 [nnzb]) of 2:4 kept values, via
    bsr_values_quantize_fp8_24."""
    _check_tensor(Vc, "Vc", (p.nnzb, p.b, p.b // 2), p.device)
    if out is None:
        out = (torch.empty((p.nnzb, p.b, p.b // 2), dtype=torch.uint8, device=Vc.device),
               torch.empty((p.nnzb,), dtype=torch.int32, device=Vc.device))
    Vc8, se = out
    _check_raw(Vc8, "Vc8", (p.nnzb, p.b, p.b // 2), torch.uint8, p.device)
    _check_raw(se, "se", (p.nnzb,), torch.int32, p.device)
    _lib.check(lib().bsr_values_quantize_fp8_24(p.handle, _ptr(Vc), _ptr(Vc8), _ptr(se), _stream(p.device)),
               "bsr_values_quantize_fp8_24")
    return Vc8, se


def linear_fwd_fp8_24(p: Pattern, X: torch.Tensor, Vc8: torch.Tensor, se: torch.Tensor, mt: torch.Tensor,
                      bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X . W~^T + bias with 2:4 blocks of fp8 kept values, via bsr_linear_fwd_fp8_24."""
    M = X.shape[0]
    _check_tensor(X, "X", (M, p.K), p.device)
    _check_raw(Vc8, "Vc8", (p.nnzb, p.b, p.b // 2), torch.uint8, p.device)
    _check_raw(se, "se", (p.nnzb,), torch.int32, p.device)
    _check_raw(mt, "meta", (p.nnzb, p.b, p.b // 16), torch.int16, p.device)
    if bias is not None:
        _check_tensor(bias, "bias", (p.N,), p.device)
    if out is None:
        out = torch.empty((M, p.N), dtype=torch.bfloat16, device=X.device)
    _check_tensor(out, "out", (M, p.N), p.device)
    _lib.check(lib().bsr_linear_fwd_fp8_24(p.handle, _ptr(X), M, _ptr(Vc8), _ptr(se), _ptr(mt), _ptr(bias),
                                           _ptr(out), _stream(p.device)), "bsr_linear_fwd_fp8_24")
    return out


def linear_fwd_small_m_csr(N: int, K: int, b: int, row_ptr: torch.Tensor, col_idx: torch.Tensor, X: torch.Tensor,
                           V: torch.Tensor, bias: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X . W~^T + bias for M <= 16 rows from device CSR metadata (e.g. meta_rebuild's), via
    bsr_linear_fwd_small_m_csr. The capacity passed is min(len(col_idx), len(V)): blocks at CSR
    positions at or past it are dropped (the truncation of a mask rebuilt past its capacity)."""
    M = X.shape[0]
    d = X.device.index
    _check_tensor(X, "X", (M, K), d)
    if V.dtype != torch.bfloat16 or not V.is_contiguous() or V.shape[1:] != (b, b):
        raise ValueError("V must be a contiguous bf16 [n, b, b] tensor")
    if col_idx.dtype != torch.int32 or row_ptr.dtype != torch.int32:
        raise TypeError("row_ptr and col_idx must be int32")
    cap = min(int(col_idx.numel()), int(V.shape[0]))
    if bias is not None:
        _check_tensor(bias, "bias", (N,), d)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    _check_tensor(out, "out", (M, N), d)
    _lib.check(lib().bsr_linear_fwd_small_m_csr(N, K, b, _ptr(row_ptr), _ptr(col_idx), cap, _ptr(X), M, _ptr(V),
                                                _ptr(bias), _ptr(out), torch.cuda.current_stream(d).cuda_stream),
               "bsr_linear_fwd_small_m_csr")
    return out
