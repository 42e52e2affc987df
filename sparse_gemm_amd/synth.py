"""Seeded synthetic inputs for the block-sparse linear layer.

This module only draws random inputs: block masks and the bf16 tensors X, V
(block values), bias and dY. It holds none of the layer's arithmetic, so both
the fp64 oracle (tests) and the HIP path consume exactly the same inputs.

The five workload shapes (sizes, block sizes, densities, the Zipf row mix) are
this project's benchmark configurations; the pages fix none of them. What the
pages do fix is the layer they exercise: a drop-in nn.Linear with a density
argument whose block pattern is chosen once at initialisation
(pytorch_block_sparse summary page, "Block-Sparse Implementation and Usage",
"Future Development Roadmap"), and the random choice of kept blocks (the
"Random" criterion of the pytorch/ao sparsity README, Table 4.2).

Random streams: one integer seed per workload; stream k of the seed is
``numpy.random.default_rng([seed, k])`` with k = 0 pattern, 1 X, 2 V, 3 bias,
4 dY, 5 a dense weight (dense-to-BSR conversion), 6 its per-block scales. Values are drawn for nonzero blocks only, in CSR order (row-major over
the block grid). Normal draws are fp32 and are rounded to bf16 with
round-to-nearest-even (``torch.Tensor.to(torch.bfloat16)``).
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional

import numpy as np
import torch

STREAM_PATTERN, STREAM_X, STREAM_V, STREAM_BIAS, STREAM_DY = 0, 1, 2, 3, 4
STREAM_W, STREAM_W_SCALE = 5, 6


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    b: int
    density: float
    pattern: str          # "uniform" or "zipf"
    bias: bool
    ops: tuple            # subset of ("fwd", "dx", "dw")
    zipf_s: float = 1.1

    @property
    def R(self) -> int:
        return self.N // self.b

    @property
    def C(self) -> int:
        return self.K // self.b

    def with_m(self, M: int) -> "Workload":
        return dataclasses.replace(self, M=M)


# The five reference workloads, keyed 1..5 in the order they are listed.
WORKLOADS = {
    1: Workload("tiny_fwd_128x256x256_b32_d0.5", 128, 256, 256, 32, 0.5, "uniform", True, ("fwd",)),
    2: Workload("bert_base_ffn_up_4096x768x3072_b32_d0.25", 4096, 768, 3072, 32, 0.25, "uniform", False,
                ("fwd", "dx", "dw")),
    3: Workload("square_8192x4096x4096_b32_d0.10", 8192, 4096, 4096, 32, 0.10, "uniform", False,
                ("fwd", "dx", "dw")),
    4: Workload("decode_8x4096x14336_b64_d0.5", 8, 4096, 14336, 64, 0.5, "uniform", False, ("fwd",)),
    5: Workload("zipf_16384x4096x11008_b32_d0.30", 16384, 4096, 11008, 32, 0.30, "zipf", False,
                ("fwd", "dx", "dw")),
}


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def uniform_mask(R: int, C: int, density: float, g: np.random.Generator) -> np.ndarray:
    """Exactly floor(density*R*C + 0.5) distinct block positions, drawn without
    replacement over the whole R x C grid (not a fixed count per row)."""
    nnzb = int(math.floor(density * R * C + 0.5))
    nnzb = max(0, min(nnzb, R * C))
    mask = np.zeros(R * C, dtype=np.uint8)
    if nnzb:
        mask[g.choice(R * C, size=nnzb, replace=False)] = 1
    return mask.reshape(R, C)


def zipf_row_counts(R: int, C: int, density: float, s: float, g: np.random.Generator) -> np.ndarray:
    """Per-row block counts: i.i.d. Zipf(s) draws, rescaled by one factor so
    that the counts, clipped to [1, C], sum to exactly round(density*R*C).

    The scale factor is found by bisection on the clipped continuous sum; the
    floors are then topped up one block each, in order of descending
    fractional part (ties to the lower row), never past C.
    """
    target = int(round(density * R * C))
    target = max(R, min(target, R * C))
    z = g.zipf(s, size=R).astype(np.float64)

    def total(lam: float) -> float:
        return float(np.clip(lam * z, 1.0, C).sum())

    lo, hi = 0.0, 1.0
    while total(hi) < target:
        hi *= 2.0
    for _ in range(300):
        mid = 0.5 * (lo + hi)
        if total(mid) < target:
            lo = mid
        else:
            hi = mid
    x = np.clip(lo * z, 1.0, C)
    n = np.floor(x).astype(np.int64)
    left = target - int(n.sum())
    frac = x - n
    while left > 0:
        order = sorted((r for r in range(R) if n[r] < C), key=lambda r: (-frac[r], r))
        for r in order[:left]:
            n[r] += 1
            frac[r] = 0.0
        left = target - int(n.sum())
    return n


def zipf_mask(R: int, C: int, density: float, s: float, g: np.random.Generator) -> np.ndarray:
    counts = zipf_row_counts(R, C, density, s, g)
    mask = np.zeros((R, C), dtype=np.uint8)
    for r in range(R):
        mask[r, g.choice(C, size=int(counts[r]), replace=False)] = 1
    return mask


def block_mask(w: Workload, seed: int = 0) -> np.ndarray:
    g = rng(seed, STREAM_PATTERN)
    if w.pattern == "uniform":
        return uniform_mask(w.R, w.C, w.density, g)
    if w.pattern == "zipf":
        return zipf_mask(w.R, w.C, w.density, w.zipf_s, g)
    raise ValueError(f"unknown pattern kind {w.pattern!r}")


def to_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def normal_bf16(shape, std: float, seed: int, stream: int) -> torch.Tensor:
    a = rng(seed, stream).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return to_bf16(a)


def activations(M: int, K: int, seed: int, stream: int = STREAM_X) -> torch.Tensor:
    """[M, K] bf16 ~ N(0, 1). The first M' rows do not depend on M."""
    return normal_bf16((M, K), 1.0, seed, stream)


def block_values(nnzb: int, b: int, seed: int) -> torch.Tensor:
    """[nnzb, b, b] bf16 ~ N(0, 0.02^2), one b x b block per nonzero, CSR order."""
    return normal_bf16((nnzb, b, b), 0.02, seed, STREAM_V)


def bias_vector(N: int, seed: int) -> torch.Tensor:
    return normal_bf16((N,), 0.02, seed, STREAM_BIAS)


def grad_output(M: int, N: int, seed: int) -> torch.Tensor:
    return normal_bf16((M, N), 1.0, seed, STREAM_DY)


def dense_weight(N: int, K: int, seed: int, b: Optional[int] = None) -> torch.Tensor:
    """A dense [N, K] bf16 weight ~ N(0, 0.02^2). With a block size b, every b x b block is
    also multiplied by its own factor exp(g), g ~ N(0, 1), before the rounding to bf16, so
    block magnitudes differ the way a trained layer's do (seeded; no trained weights)."""
    a = rng(seed, STREAM_W).standard_normal(size=(N, K), dtype=np.float32) * np.float32(0.02)
    if b is not None:
        f = np.exp(rng(seed, STREAM_W_SCALE).standard_normal(size=(N // b, K // b))).astype(np.float32)
        a *= np.repeat(np.repeat(f, b, axis=0), b, axis=1)
    return to_bf16(a)


def make_inputs(w: Workload, seed: int = 0, mask: Optional[np.ndarray] = None, with_dy: Optional[bool] = None):
    """All inputs of one workload on the host: mask, X, V, bias (or None), dY (or None)."""
    if mask is None:
        mask = block_mask(w, seed)
    nnzb = int(mask.sum())
    X = activations(w.M, w.K, seed)
    V = block_values(nnzb, w.b, seed)
    bias = bias_vector(w.N, seed) if w.bias else None
    if with_dy is None:
        with_dy = ("dx" in w.ops) or ("dw" in w.ops)
    dY = grad_output(w.M, w.N, seed) if with_dy else None
    return dict(mask=mask, X=X, V=V, bias=bias, dY=dY)


def mask_digest(mask: np.ndarray) -> str:
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    h = hashlib.sha256()
    h.update(np.asarray(m.shape, dtype=np.int64).tobytes())
    h.update(m.tobytes())
    return h.hexdigest()


def row_histogram(mask: np.ndarray) -> dict:
    counts = mask.sum(axis=1).astype(np.int64)
    C = mask.shape[1]
    return dict(min=int(counts.min()) if counts.size else 0, max=int(counts.max()) if counts.size else 0,
                median=float(np.median(counts)) if counts.size else 0.0,
                full_rows=int((counts == C).sum()), single_rows=int((counts == 1).sum()),
                empty_rows=int((counts == 0).sum()))
