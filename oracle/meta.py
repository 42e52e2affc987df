"""Block-pattern metadata by direct scan of the block mask (oracle side).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). Written independently of
the HIP library's pattern builder, which the tests compare against this bit
for bit.

Definitions (pytorch/ao sparsity README, Table 4.1): CSR/CSC store an index
pointer (IndexPtr: where each row's / column's entries start, from row 0),
the indices of the entries, and their data; BSR does the same with dense
blocks as the entries. Orders inside a row / column are not fixed by the
page; this oracle takes the canonical ascending order.

  row_ptr[r]  : index of the first nonzero block of block row r (CSR order);
                row_ptr[R] = nnzb.
  col_idx[i]  : block column of the i-th nonzero block in CSR order.
  col_ptr[c]  : index of the first nonzero block of block column c in CSC
                order; col_ptr[C] = nnzb.
  row_idx[j]  : block row of the j-th nonzero block in CSC order.
  perm[j]     : CSR index of the j-th nonzero block in CSC order.
"""
from __future__ import annotations

import numpy as np


def scan(mask) -> dict:
    """Plain loops over a (R, C) block mask (nonzero = kept block)."""
    mask = np.asarray(mask)
    R, C = mask.shape
    row_ptr = [0]
    col_idx = []
    for r in range(R):                       # row-major scan
        for c in range(C):
            if mask[r, c]:
                col_idx.append(c)
        row_ptr.append(len(col_idx))

    col_ptr = [0]
    row_idx = []
    for c in range(C):                       # column-major scan
        for r in range(R):
            if mask[r, c]:
                row_idx.append(r)
        col_ptr.append(len(row_idx))

    perm = []
    for c in range(C):
        for j in range(col_ptr[c], col_ptr[c + 1]):
            r = row_idx[j]
            found = -1
            for i in range(row_ptr[r], row_ptr[r + 1]):   # search row r's column list
                if col_idx[i] == c:
                    found = i
                    break
            assert found >= 0
            perm.append(found)

    as_i32 = lambda v: np.asarray(v, dtype=np.int32)
    return dict(row_ptr=as_i32(row_ptr), col_idx=as_i32(col_idx), col_ptr=as_i32(col_ptr),
                row_idx=as_i32(row_idx), perm=as_i32(perm), R=R, C=C, nnzb=len(col_idx))


def dense_weight(row_ptr, col_idx, V, N: int, K: int, b: int) -> np.ndarray:
    """W~ [N, K] fp64: zero except block (r, col_idx[i]) = V[i]."""
    V = np.asarray(V, dtype=np.float64)
    W = np.zeros((N, K), dtype=np.float64)
    R = N // b
    for r in range(R):
        for i in range(int(row_ptr[r]), int(row_ptr[r + 1])):
            c = int(col_idx[i])
            W[r * b:(r + 1) * b, c * b:(c + 1) * b] = V[i]
    return W
