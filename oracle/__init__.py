"""fp64 CPU oracle of the block-sparse linear layer.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and
the benchmark's ``cpu_baseline`` leg may import this package. It shares no
code with the HIP library (``sparse_gemm_amd``) and never imports it.

Parts:
  oracle.c  plain fp64 loops over the nonzero blocks (forward, input grad,
            weight grad on the pattern, bias grad), each output paired with
            S = sum of |products| for the tolerance rule;
  meta.py   CSR / CSC / perm metadata by direct scan of the block mask;
  brute.py  exact Fraction brute force over the dense zero-filled weight;
  oracle.c  also: fp8 (OCP E4M3) block values with a power-of-two scale per
            block (quantise, dequantise); 2:4 sparsity inside each kept
            block (compress by magnitude, decompress);
  convert.py dense <-> BSR conversion and block-magnitude pattern selection
            (block norms from oracle.c, top-k by a plain sort, gather and
            scatter of blocks by plain loops).

The acceptance rule for a bf16 result g against the fp64 value o is
|g - o| <= 4e-3 * S(o), and g == o exactly where S(o) == 0.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import meta  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")
TOL = 4e-3

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no FP contraction)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
               "-std=c11", "-Wall", "-o", tmp, SRC_PATH, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, P = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.oracle_fwd.argtypes = [i64, i32, i32, i32, P, P, P, P, P, P, P]
        L.oracle_dx.argtypes = [i64, i32, i32, i32, P, P, P, P, P, P]
        L.oracle_dw.argtypes = [i64, i32, i32, i32, P, P, P, P, P, i32, P, P]
        L.oracle_db.argtypes = [i64, i32, P, P, P]
        L.oracle_block_norms.argtypes = [i32, i32, i32, i32, P, P]
        L.oracle_quantize_fp8.argtypes = [i32, i32, P, P, P]
        L.oracle_dequantize_fp8.argtypes = [i32, i32, P, P, P]
        L.oracle_compress_24.argtypes = [i32, i32, P, P, P]
        L.oracle_decompress_24.argtypes = [i32, i32, P, P, P]
        L.oracle_e4m3_value.argtypes, L.oracle_e4m3_value.restype = [ctypes.c_uint8], ctypes.c_double
        L.oracle_e4m3_encode.argtypes, L.oracle_e4m3_encode.restype = [ctypes.c_double], ctypes.c_uint8
        for f in (L.oracle_fwd, L.oracle_dx, L.oracle_dw, L.oracle_db, L.oracle_block_norms, L.oracle_quantize_fp8,
                  L.oracle_dequantize_fp8, L.oracle_compress_24, L.oracle_decompress_24):
            f.restype = None
        L.oracle_max_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes, L.oracle_set_threads.restype = [ctypes.c_int], None
        _lib = L
    return _lib


def _f64(a) -> np.ndarray:
    """Exact widening to a contiguous fp64 numpy array (torch bf16/fp32 or numpy)."""
    if hasattr(a, "detach"):
        a = a.detach().to("cpu")
        import torch
        a = a.to(torch.float64).numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def fwd(X, row_ptr, col_idx, V, N: int, b: int, bias=None, want_s: bool = True):
    """Y = X . W~^T + bias, and S. Returns (Y, S) as fp64 [M, N] arrays (S None if not wanted)."""
    X, V = _f64(X), _f64(V)
    bias = None if bias is None else _f64(bias)
    row_ptr, col_idx = _i32(row_ptr), _i32(col_idx)
    M, K = X.shape
    Y = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64) if want_s else None
    lib().oracle_fwd(M, N, K, b, _p(row_ptr), _p(col_idx), _p(X), _p(V), _p(bias), _p(Y), _p(S))
    return Y, S


def dx(dY, row_ptr, col_idx, V, K: int, b: int, want_s: bool = True):
    """dX = dY . W~ (walking CSR), and S."""
    dY, V = _f64(dY), _f64(V)
    row_ptr, col_idx = _i32(row_ptr), _i32(col_idx)
    M, N = dY.shape
    dX = np.empty((M, K), dtype=np.float64)
    S = np.empty((M, K), dtype=np.float64) if want_s else None
    lib().oracle_dx(M, N, K, b, _p(row_ptr), _p(col_idx), _p(dY), _p(V), _p(dX), _p(S))
    return dX, S


def dw(dY, X, row_ptr, col_idx, b: int, blocks=None, want_s: bool = True):
    """dV for the listed block indices (all, in CSR order, if None), and S."""
    dY, X = _f64(dY), _f64(X)
    row_ptr, col_idx = _i32(row_ptr), _i32(col_idx)
    M, N = dY.shape
    K = X.shape[1]
    blk = None if blocks is None else _i32(blocks)
    nb = int(row_ptr[-1]) if blk is None else int(blk.size)
    dV = np.empty((nb, b, b), dtype=np.float64)
    S = np.empty((nb, b, b), dtype=np.float64) if want_s else None
    lib().oracle_dw(M, N, K, b, _p(row_ptr), _p(col_idx), _p(dY), _p(X), _p(blk), nb, _p(dV), _p(S))
    return dV, S


def db(dY, want_s: bool = True):
    dY = _f64(dY)
    M, N = dY.shape
    out = np.empty((N,), dtype=np.float64)
    S = np.empty((N,), dtype=np.float64) if want_s else None
    lib().oracle_db(M, N, _p(dY), _p(out), _p(S))
    return out, S


def block_norms(W, b: int, kind: int = 1) -> np.ndarray:
    """Per-block magnitude of a dense weight W [N, K]: kind 1 = L1, kind 2 = squared L2.
    Returns an fp64 [N/b, K/b] array (summation order stated in oracle.c)."""
    if kind not in (1, 2):
        raise ValueError("kind must be 1 (L1) or 2 (squared L2)")
    W = _f64(W)
    N, K = W.shape
    out = np.empty((N // b, K // b), dtype=np.float64)
    lib().oracle_block_norms(N, K, b, kind, _p(W), _p(out))
    return out


def e4m3_value(code: int) -> float:
    return float(lib().oracle_e4m3_value(int(code)))


def e4m3_encode(x: float) -> int:
    return int(lib().oracle_e4m3_encode(float(x)))


def quantize_fp8(V):
    """(codes uint8, scale exponents int32 [nnzb]) of per-block values V [nnzb, ...] (one scale per
    leading index: dense blocks [nnzb, b, b], or the kept values of 2:4 blocks [nnzb, b, b/2])."""
    V = _f64(V)
    nnzb = V.shape[0]
    n = int(np.prod(V.shape[1:]))
    codes = np.empty(V.shape, dtype=np.uint8)
    se = np.empty((nnzb,), dtype=np.int32)
    lib().oracle_quantize_fp8(nnzb, n, _p(V), _p(codes), _p(se))
    return codes, se


def dequantize_fp8(codes, se) -> np.ndarray:
    """fp64 values of the same shape as codes: code value * 2^se per leading index."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    se = _i32(se)
    nnzb = codes.shape[0]
    n = int(np.prod(codes.shape[1:]))
    out = np.empty(codes.shape, dtype=np.float64)
    lib().oracle_dequantize_fp8(nnzb, n, _p(codes), _p(se), _p(out))
    return out


def compress_24(V):
    """(Vc fp64 [nnzb, b, b/2], meta uint16 [nnzb, b, b/16]): the two largest magnitudes of every
    group of 4 columns of every block row (ties to the lower position), see oracle.c."""
    V = _f64(V)
    nnzb, b, _ = V.shape
    Vc = np.empty((nnzb, b, b // 2), dtype=np.float64)
    meta_ = np.empty((nnzb, b, b // 16), dtype=np.uint16)
    lib().oracle_compress_24(nnzb, b, _p(V), _p(Vc), _p(meta_))
    return Vc, meta_


def decompress_24(Vc, meta_) -> np.ndarray:
    """fp64 [nnzb, b, b] dense blocks from the compressed form."""
    Vc = _f64(Vc)
    meta_ = np.ascontiguousarray(meta_, dtype=np.uint16)
    nnzb, b, _ = Vc.shape
    out = np.empty((nnzb, b, b), dtype=np.float64)
    lib().oracle_decompress_24(nnzb, b, _p(Vc), _p(meta_), _p(out))
    return out


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def set_threads(n: int) -> None:
    """Threads of the OpenMP loops (results are the same for any count)."""
    lib().oracle_set_threads(int(n))


def tolerance_check(g, ref: np.ndarray, S: np.ndarray, tol: float = TOL) -> dict:
    """Acceptance rule: |g - ref| <= tol * S elementwise; exact where S == 0.

    Returns the worst ratio |g - ref| / S over S > 0, the count of violations
    and the count of elements checked.
    """
    g = _f64(g)
    err = np.abs(g - ref)
    pos = S > 0
    viol = int(np.count_nonzero(err[pos] > tol * S[pos])) + int(np.count_nonzero(err[~pos] != 0))
    viol += int(np.count_nonzero(~np.isfinite(g)))
    ratio = float(np.max(err[pos] / S[pos])) if np.any(pos) else 0.0
    return dict(max_ratio=ratio, violations=viol, checked=int(g.size))
