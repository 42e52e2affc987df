"""BlockSparseLinear: a drop-in nn.Linear whose weight keeps a fixed pattern of dense blocks.

pytorch_block_sparse summary page, "Block-Sparse Implementation and Usage": the layer
replaces torch.nn.Linear and takes a density at construction; "Future Development
Roadmap": the pattern is fixed at initialisation. The pattern here is drawn uniformly at
random over the block grid (the "Random" pruning criterion of the pytorch/ao sparsity
README, Table 4.2) unless a block mask is given. Forward, input gradient and weight
gradient run in the HIP library (bsr_linear_fwd / _bwd_input / _bwd_weight).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch
from torch import nn

from . import binding
from .binding import Pattern


class _BsrLinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x2d: torch.Tensor, values: torch.Tensor, bias: Optional[torch.Tensor], pattern: Pattern):
        ctx.pattern = pattern
        ctx.has_bias = bias is not None
        ctx.save_for_backward(x2d, values)
        return binding.linear_fwd(pattern, x2d, values, bias)

    @staticmethod
    def backward(ctx, dY: torch.Tensor):
        x2d, values = ctx.saved_tensors
        p = ctx.pattern
        dY = dY.to(torch.bfloat16).contiguous()
        dX = dV = db = None
        if ctx.needs_input_grad[0]:
            dX = binding.linear_bwd_input(p, dY, values)
        if ctx.needs_input_grad[1] or (ctx.has_bias and ctx.needs_input_grad[2]):
            dV, db = binding.linear_bwd_weight(p, dY, x2d, want_dbias=ctx.has_bias and ctx.needs_input_grad[2])
            if not ctx.needs_input_grad[1]:
                dV = None
        return dX, dV, db, None


def bsr_linear(x: torch.Tensor, pattern: Pattern, values: torch.Tensor, bias: Optional[torch.Tensor] = None):
    """Functional form: x [..., K] -> [..., N]."""
    lead = x.shape[:-1]
    x2d = x.reshape(-1, x.shape[-1]).to(torch.bfloat16).contiguous()
    y = _BsrLinearFn.apply(x2d, values, bias, pattern)
    return y.reshape(*lead, pattern.N)


def random_block_mask(out_features: int, in_features: int, block_size: int, density: float, seed: int) -> np.ndarray:
    """Seeded uniform block mask with exactly floor(density*R*C + 0.5) kept blocks."""
    R, C = out_features // block_size, in_features // block_size
    nnzb = max(0, min(R * C, int(math.floor(density * R * C + 0.5))))
    g = np.random.default_rng([int(seed), 0])
    mask = np.zeros(R * C, dtype=np.uint8)
    if nnzb:
        mask[g.choice(R * C, size=nnzb, replace=False)] = 1
    return mask.reshape(R, C)


class BlockSparseLinear(nn.Module):
    """y = x W^T + b with W [out, in] stored as BSR blocks of size block_size (32 or 64)."""

    def __init__(self, in_features: int, out_features: int, bias: bool = True, density: float = 0.5,
                 block_size: int = 32, seed: int = 0, mask: Optional[np.ndarray] = None, device=None):
        super().__init__()
        if in_features % block_size or out_features % block_size:
            raise ValueError("in_features and out_features must be multiples of block_size")
        self.in_features, self.out_features, self.block_size = in_features, out_features, block_size
        if mask is None:
            mask = random_block_mask(out_features, in_features, block_size, density, seed)
        mask = np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
        device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        with torch.cuda.device(device):
            self.pattern = Pattern.from_mask(mask, out_features, in_features, block_size)
        meta = self.pattern.export()
        self.register_buffer("row_ptr", torch.from_numpy(meta["row_ptr"].copy()), persistent=True)
        self.register_buffer("col_idx", torch.from_numpy(meta["col_idx"].copy()), persistent=True)
        self.values = nn.Parameter(torch.empty((self.pattern.nnzb, block_size, block_size), dtype=torch.bfloat16,
                                               device=device))
        self.bias = nn.Parameter(torch.empty((out_features,), dtype=torch.bfloat16, device=device)) if bias else None
        self.reset_parameters()

    @property
    def density(self) -> float:
        return self.pattern.nnzb / max(1, self.pattern.R * self.pattern.C)

    def reset_parameters(self) -> None:
        bound = 1.0 / math.sqrt(max(1, self.in_features))
        with torch.no_grad():
            self.values.uniform_(-bound, bound)
            if self.bias is not None:
                self.bias.uniform_(-bound, bound)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return bsr_linear(x, self.pattern, self.values, self.bias)

    def block_mask(self) -> np.ndarray:
        return self._mask_of(self.pattern)

    @torch.no_grad()
    def to_dense(self) -> torch.Tensor:
        """Dense weight [out, in] with zeros outside the kept blocks (the hand-off format of
        the pytorch/ao sparsity README, workflow section), written by bsr_values_to_dense."""
        return binding.values_to_dense(self.pattern, self.values.detach().contiguous())

    @classmethod
    @torch.no_grad()
    def from_dense(cls, linear: nn.Linear, block_mask: np.ndarray, block_size: int = 32) -> "BlockSparseLinear":
        """Keep the blocks of a dense nn.Linear that block_mask selects (bsr_dense_to_values)."""
        W = linear.weight.detach().to(torch.bfloat16).contiguous()
        out_f, in_f = W.shape
        m = cls(in_f, out_f, bias=linear.bias is not None, block_size=block_size, mask=block_mask, device=W.device)
        binding.dense_to_values(m.pattern, W, out=m.values.data)
        if linear.bias is not None:
            m.bias.copy_(linear.bias.detach().to(torch.bfloat16))
        return m

    @classmethod
    @torch.no_grad()
    def from_dense_by_magnitude(cls, linear: nn.Linear, density: float, block_size: int = 32,
                                norm: int = binding.NORM_L1) -> "BlockSparseLinear":
        """Magnitude pruning at block granularity (pytorch/ao sparsity README, Table 4.2: drop
        the lowest norms, L1 by default; layer-local scope): keep the floor(density*R*C + 0.5)
        blocks of largest norm of the dense weight, then read them into BSR."""
        W = linear.weight.detach().to(torch.bfloat16).contiguous()
        out_f, in_f = W.shape
        R, C = out_f // block_size, in_f // block_size
        keep = max(0, min(R * C, int(math.floor(density * R * C + 0.5))))
        with torch.cuda.device(W.device):
            p = Pattern.from_dense(W, block_size, keep, norm)
        m = cls(in_f, out_f, bias=linear.bias is not None, block_size=block_size, mask=cls._mask_of(p),
                device=W.device)
        p.close()
        binding.dense_to_values(m.pattern, W, out=m.values.data)
        if linear.bias is not None:
            m.bias.copy_(linear.bias.detach().to(torch.bfloat16))
        return m

    @staticmethod
    def _mask_of(p: Pattern) -> np.ndarray:
        meta = p.export()
        mask = np.zeros((p.R, p.C), dtype=np.uint8)
        for r in range(p.R):
            mask[r, meta["col_idx"][meta["row_ptr"][r]:meta["row_ptr"][r + 1]]] = 1
        return mask

    def _load_from_state_dict(self, state_dict, prefix, local_metadata, strict, missing_keys, unexpected_keys,
                              error_msgs):
        """Loads the pattern (row_ptr, col_idx) with the values. When the saved pattern differs from
        the module's, the pattern is rebuilt and `values` is resized in place: the Parameter object
        stays the same, so an optimizer built earlier still updates it, but any per-parameter
        optimizer state of `values` (momentum, Adam moments) no longer matches its shape and must
        be reset by the caller."""
        rp, ci = state_dict.get(prefix + "row_ptr"), state_dict.get(prefix + "col_idx")
        if rp is not None and ci is not None:
            rp_np = rp.cpu().numpy().astype(np.int32)
            ci_np = ci.cpu().numpy().astype(np.int32)
            if not (np.array_equal(rp_np, self.row_ptr.cpu().numpy()) and
                    np.array_equal(ci_np, self.col_idx.cpu().numpy())):
                dev = self.values.device
                with torch.cuda.device(dev):
                    self.pattern = Pattern.from_csr(self.out_features, self.in_features, self.block_size, rp_np,
                                                    ci_np)
                self.row_ptr = torch.from_numpy(rp_np.copy())
                self.col_idx = torch.from_numpy(ci_np.copy())
                self.values.data = torch.empty((self.pattern.nnzb, self.block_size, self.block_size),
                                               dtype=torch.bfloat16, device=dev)
                self.values.grad = None
        super()._load_from_state_dict(state_dict, prefix, local_metadata, strict, missing_keys, unexpected_keys,
                                      error_msgs)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, block_size={self.block_size}, "
                f"density={self.density:.4f}, bias={self.bias is not None}")
