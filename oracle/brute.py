"""Exact brute force of the block-sparse linear layer on tiny inputs.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). Every value is a
fractions.Fraction, so the results are exact; the sums follow the scalar
definition over the dense zero-filled weight (pytorch/ao sparsity README,
workflow section: sparse and dense matmul with zeros in the missing places
are numerically equivalent), and the weight gradient is the dense gradient
restricted to the kept blocks (README's out-of-place mask update,
"dW' = dW (Mask)").

Inputs are nested lists (or arrays) of numbers convertible to Fraction;
`mask` is the (R, C) block mask and `W` the dense [N, K] weight (entries
outside kept blocks are ignored, i.e. treated as 0).
"""
from __future__ import annotations

from fractions import Fraction


def _F(a):
    return [[Fraction(float(v)) if not isinstance(v, Fraction) else v for v in row] for row in a]


def masked_weight(W, mask, b):
    W = _F(W)
    N, K = len(W), len(W[0])
    return [[W[n][k] if mask[n // b][k // b] else Fraction(0) for k in range(K)] for n in range(N)]


def forward(X, W, mask, b, bias=None):
    """Y[m][n] = sum_k X[m][k] * Wm[n][k] + bias[n]."""
    X = _F(X)
    Wm = masked_weight(W, mask, b)
    M, K, N = len(X), len(X[0]), len(Wm)
    Y = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += X[m][k] * Wm[n][k]
            if bias is not None:
                acc += Fraction(float(bias[n]))
            row.append(acc)
        Y.append(row)
    return Y


def grad_input(dY, W, mask, b):
    """dX[m][k] = sum_n dY[m][n] * Wm[n][k]."""
    dY = _F(dY)
    Wm = masked_weight(W, mask, b)
    M, N, K = len(dY), len(Wm), len(Wm[0])
    return [[sum((dY[m][n] * Wm[n][k] for n in range(N)), Fraction(0)) for k in range(K)] for m in range(M)]


def grad_weight_dense(dY, X, mask, b):
    """(dY^T X) with entries outside kept blocks set to 0, as a dense [N, K]."""
    dY, X = _F(dY), _F(X)
    M, N, K = len(dY), len(dY[0]), len(X[0])
    G = []
    for n in range(N):
        row = []
        for k in range(K):
            if mask[n // b][k // b]:
                row.append(sum((dY[m][n] * X[m][k] for m in range(M)), Fraction(0)))
            else:
                row.append(Fraction(0))
        G.append(row)
    return G


def grad_bias(dY):
    dY = _F(dY)
    return [sum((dY[m][n] for m in range(len(dY))), Fraction(0)) for n in range(len(dY[0]))]
