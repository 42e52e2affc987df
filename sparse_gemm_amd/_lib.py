"""ctypes binding of libbsr_linear.so (the C ABI in include/*.h).

Argument marshalling only: every step of the computation runs in the library's HIP
kernels. There is no CPU fallback; if the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# BSR_LIB_PATH selects another build of the same library (tuning experiments).
LIB_PATH = os.environ.get("BSR_LIB_PATH") or os.path.join(_HERE, "libbsr_linear.so")

# Names and codes of include/bsr_linear.h.
STATUS = {0: "BSR_OK", 1: "BSR_ERR_INVALID_ARG", 2: "BSR_ERR_UNSUPPORTED", 3: "BSR_ERR_MISALIGNED",
          4: "BSR_ERR_WORKSPACE_TOO_SMALL", 5: "BSR_ERR_HIP", 6: "BSR_ERR_OUT_OF_MEMORY",
          7: "BSR_ERR_NO_DEVICE_DATA"}
EXPORTS = ("bsr_abi_version", "bsr_pattern_create_from_mask", "bsr_pattern_create_from_csr",
           "bsr_pattern_info", "bsr_pattern_export", "bsr_pattern_destroy", "bsr_linear_fwd",
           "bsr_linear_bwd_input", "bsr_linear_bwd_weight_workspace", "bsr_linear_bwd_weight",
           "bsr_linear_bwd_weight_noalloc", "bsr_op_kernels",
           "bsr_status_string", "bsr_last_error",
           # include/bsr_convert.h
           "bsr_block_norms", "bsr_mask_topk", "bsr_pattern_create_from_dense", "bsr_dense_to_values",
           "bsr_values_to_dense",
           # include/bsr_fp8.h
           "bsr_values_quantize_fp8", "bsr_values_dequantize_fp8", "bsr_linear_fwd_fp8",
           # include/bsr_sparse24.h
           "bsr_values_compress_24", "bsr_values_decompress_24", "bsr_linear_fwd_24", "bsr_values_pack_24",
           "bsr_linear_fwd_24_image", "bsr_values_quantize_fp8_24", "bsr_linear_fwd_fp8_24",
           # include/bsr_rebuild.h
           "bsr_meta_rebuild_workspace", "bsr_meta_rebuild", "bsr_linear_fwd_small_m_csr",
           "bsr_pattern_create_device", "bsr_pattern_rebuild", "bsr_pattern_device_arrays")


class BsrError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")


_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library (built by sparse_gemm_amd.build); raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m sparse_gemm_amd.build` "
                          "(there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, P, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    PP = ctypes.POINTER(ctypes.c_void_p)
    L.bsr_abi_version.argtypes, L.bsr_abi_version.restype = [], i32
    L.bsr_pattern_create_from_mask.argtypes = [i32, i32, i32, P, i32, PP]
    L.bsr_pattern_create_from_csr.argtypes = [i32, i32, i32, i32, P, P, i32, PP]
    L.bsr_pattern_info.argtypes = [P, P, P, P, P]
    L.bsr_pattern_export.argtypes = [P, P, P, P, P, P]
    L.bsr_pattern_destroy.argtypes, L.bsr_pattern_destroy.restype = [P], None
    L.bsr_linear_fwd.argtypes = [P, P, i64, P, P, P, P]
    L.bsr_linear_bwd_input.argtypes = [P, P, i64, P, P, P]
    L.bsr_linear_bwd_weight_workspace.argtypes, L.bsr_linear_bwd_weight_workspace.restype = [P, i64], sz
    L.bsr_op_kernels.argtypes, L.bsr_op_kernels.restype = [P, i32, i64, ctypes.c_char_p, i32], i32
    L.bsr_linear_bwd_weight.argtypes = [P, P, P, i64, P, P, P, sz, P]
    L.bsr_linear_bwd_weight_noalloc.argtypes = [P, P, P, i64, P, P, P]
    L.bsr_block_norms.argtypes = [i32, i32, i32, P, i32, P, P]
    L.bsr_mask_topk.argtypes = [i32, i32, P, i64, P]
    L.bsr_pattern_create_from_dense.argtypes = [i32, i32, i32, P, i32, i64, P, PP]
    L.bsr_dense_to_values.argtypes = [P, P, P, P]
    L.bsr_values_to_dense.argtypes = [P, P, P, P]
    L.bsr_values_quantize_fp8.argtypes = [P, P, P, P, P]
    L.bsr_values_dequantize_fp8.argtypes = [P, P, P, P, P]
    L.bsr_linear_fwd_fp8.argtypes = [P, P, i64, P, P, P, P, P]
    L.bsr_values_compress_24.argtypes = [P, P, P, P, P]
    L.bsr_values_decompress_24.argtypes = [P, P, P, P, P]
    L.bsr_linear_fwd_24.argtypes = [P, P, i64, P, P, P, P, P]
    L.bsr_values_pack_24.argtypes = [P, P, P, P, P]
    L.bsr_values_quantize_fp8_24.argtypes = [P, P, P, P, P]
    L.bsr_linear_fwd_fp8_24.argtypes = [P, P, i64, P, P, P, P, P, P]
    L.bsr_linear_fwd_24_image.argtypes = [P, P, i64, P, P, P, P]
    L.bsr_meta_rebuild_workspace.argtypes, L.bsr_meta_rebuild_workspace.restype = [i32, i32], sz
    L.bsr_meta_rebuild.argtypes = [i32, i32, P, P, P, P, P, P, i32, P, P, sz, P]
    L.bsr_linear_fwd_small_m_csr.argtypes = [i32, i32, i32, P, P, i32, P, i64, P, P, P, P]
    L.bsr_pattern_create_device.argtypes = [i32, i32, i32, i32, PP]
    L.bsr_pattern_rebuild.argtypes = [P, P, P]
    L.bsr_pattern_device_arrays.argtypes = [P, PP, PP, PP, PP, PP, PP]
    for f in ("bsr_pattern_create_from_mask", "bsr_pattern_create_from_csr", "bsr_pattern_info",
              "bsr_pattern_export", "bsr_linear_fwd", "bsr_linear_bwd_input", "bsr_linear_bwd_weight",
              "bsr_linear_bwd_weight_noalloc",
              "bsr_block_norms", "bsr_mask_topk", "bsr_pattern_create_from_dense", "bsr_dense_to_values",
              "bsr_values_to_dense",
           # include/bsr_fp8.h
           "bsr_values_quantize_fp8", "bsr_values_dequantize_fp8", "bsr_linear_fwd_fp8",
           # include/bsr_sparse24.h
           "bsr_values_compress_24", "bsr_values_decompress_24", "bsr_linear_fwd_24", "bsr_values_pack_24",
           "bsr_linear_fwd_24_image", "bsr_values_quantize_fp8_24", "bsr_linear_fwd_fp8_24",
           # include/bsr_rebuild.h
           "bsr_meta_rebuild_workspace", "bsr_meta_rebuild", "bsr_linear_fwd_small_m_csr",
           "bsr_pattern_create_device", "bsr_pattern_rebuild", "bsr_pattern_device_arrays"):
        getattr(L, f).restype = i32
    L.bsr_status_string.argtypes, L.bsr_status_string.restype = [i32], ctypes.c_char_p
    L.bsr_last_error.argtypes, L.bsr_last_error.restype = [], ctypes.c_char_p
    _lib = L
    return L


def check(status: int, where: str) -> None:
    if status != 0:
        detail = load().bsr_last_error().decode(errors="replace")
        raise BsrError(status, where, detail)
