"""Dense <-> BSR conversion and block-magnitude pattern selection (oracle side).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). Shares no code with the
HIP library.

What is computed:
  * The hand-off between a pruning front end and the sparse kernels is a dense
    weight with zeros in the missing places (pytorch/ao sparsity README,
    workflow section). values_to_dense builds that dense weight from BSR;
    dense_to_values reads the kept blocks out of a dense weight into BSR block
    order (README Table 4.1: BSR = dense blocks plus their coordinates).
  * The magnitude criterion (README Table 4.2; pytorch_block_sparse summary
    page, "Future Development Roadmap": measuring parameter usefulness to pick
    the pattern) keeps the blocks with the largest norm. topk_mask keeps the
    `keep` largest block norms of one layer (the README's local scope), ties
    going to the lower row-major block index; block_norms lives in oracle.c.

All functions copy values without arithmetic, so any dtype works; the tests
pass raw bf16 bit patterns (int16 / uint16) to compare bits.
"""
from __future__ import annotations

import numpy as np


def topk_mask(norms, keep: int) -> np.ndarray:
    """[R, C] uint8 mask of the `keep` blocks with the largest norm (ties: lower r*C + c)."""
    norms = np.asarray(norms, dtype=np.float64)
    R, C = norms.shape
    if not 0 <= keep <= R * C:
        raise ValueError("keep out of range")
    flat = norms.ravel()
    if np.isnan(flat).any():
        raise ValueError("NaN norm")
    order = sorted(range(flat.size), key=lambda i: (-flat[i], i))
    mask = np.zeros(R * C, dtype=np.uint8)
    for i in order[:keep]:
        mask[i] = 1
    return mask.reshape(R, C)


def dense_to_values(W, row_ptr, col_idx, b: int) -> np.ndarray:
    """V[i] = block (r, col_idx[i]) of the dense W, for every kept block i in CSR order."""
    W = np.asarray(W)
    R = len(row_ptr) - 1
    nnzb = int(row_ptr[R])
    V = np.empty((nnzb, b, b), dtype=W.dtype)
    for r in range(R):
        for i in range(int(row_ptr[r]), int(row_ptr[r + 1])):
            c = int(col_idx[i])
            for p in range(b):
                V[i, p, :] = W[r * b + p, c * b:(c + 1) * b]
    return V


def values_to_dense(V, row_ptr, col_idx, N: int, K: int, b: int) -> np.ndarray:
    """The dense [N, K] weight: block (r, col_idx[i]) = V[i], zero everywhere else."""
    V = np.asarray(V)
    W = np.zeros((N, K), dtype=V.dtype)
    R = len(row_ptr) - 1
    for r in range(R):
        for i in range(int(row_ptr[r]), int(row_ptr[r + 1])):
            c = int(col_idx[i])
            for p in range(b):
                W[r * b + p, c * b:(c + 1) * b] = V[i, p, :]
    return W
