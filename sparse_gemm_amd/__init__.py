"""Block-sparse linear layer on AMD MI355X (gfx950): BSR weights, bf16 MFMA kernels, C ABI.

Public names (loaded on first use, so that importing the package does not load the HIP
library):
  Pattern, linear_fwd, linear_bwd_input, linear_bwd_weight   -- sparse_gemm_amd.binding
  BlockSparseLinear, bsr_linear                              -- sparse_gemm_amd.linear
Build the library with `python -m sparse_gemm_amd.build`.
"""
__all__ = ["Pattern", "linear_fwd", "linear_bwd_input", "linear_bwd_weight", "BlockSparseLinear", "bsr_linear"]

_BINDING = {"Pattern", "linear_fwd", "linear_bwd_input", "linear_bwd_weight"}
_LINEAR = {"BlockSparseLinear", "bsr_linear"}


def __getattr__(name):
    if name in _BINDING:
        from . import binding
        return getattr(binding, name)
    if name in _LINEAR:
        from . import linear
        return getattr(linear, name)
    raise AttributeError(name)
