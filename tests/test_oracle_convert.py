"""Pins of the oracle's dense <-> BSR conversion and block-magnitude selection.

Each pin comes from the pages or the mathematics, not from re-typing the oracle:
  * a hand-worked example (tests/golden/block_norms_b2.json);
  * exact Fraction sums, and the textbook error bound of a left-to-right fp64 sum on
    inputs where the sum is not exact;
  * closed forms: a constant block, a single nonzero, power-of-two scaling;
  * a different formulation of the same quantity (reshape-and-reduce);
  * brute force over every subset for the top-k selection, and recovery of a planted
    block support;
  * round trips between the dense hand-off form (README workflow section: a dense weight
    with zeros in the missing places) and BSR (README Table 4.1), checked against a
    Kronecker-product mask and against the forward of the block-sparse layer;
  * planted mistakes in copies of the oracle must fail a pin.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import convert, meta
from sparse_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "block_norms_b2.json")) as f:
        return json.load(f)


def test_golden_norms_masks_and_bsr():
    g = _golden()
    W = np.array(g["W"], dtype=np.float64)
    b = g["b"]
    assert np.array_equal(oracle.block_norms(W, b, 1), np.array(g["l1"]))
    assert np.array_equal(oracle.block_norms(W, b, 2), np.array(g["l2sq"]))
    for case in g["masks"]:
        norms = oracle.block_norms(W, b, case["kind"])
        assert np.array_equal(convert.topk_mask(norms, case["keep"]), np.array(case["mask"])), case
    e = g["bsr_l1_keep3"]
    md = meta.scan(convert.topk_mask(oracle.block_norms(W, b, 1), 3))
    assert md["row_ptr"].tolist() == e["row_ptr"] and md["col_idx"].tolist() == e["col_idx"]
    V = convert.dense_to_values(W, md["row_ptr"], md["col_idx"], b)
    assert np.array_equal(V, np.array(e["V"], dtype=np.float64))
    D = convert.values_to_dense(V, md["row_ptr"], md["col_idx"], g["N"], g["K"], b)
    assert np.array_equal(D, np.array(e["dense"], dtype=np.float64))


def _exact_block_sums(W, b, kind):
    N, K = W.shape
    out = []
    for r in range(N // b):
        row = []
        for c in range(K // b):
            s = Fraction(0)
            for p in range(b):
                for q in range(b):
                    w = Fraction(float(W[r * b + p, c * b + q]))
                    s += abs(w) if kind == 1 else w * w
            row.append(s)
        out.append(row)
    return out


@pytest.mark.parametrize("kind", [1, 2])
def test_norms_exact_on_small_integers(kind):
    """Integer entries in [-8, 8]: every partial sum is an integer far below 2^53, so the
    fp64 result must equal the exact sum."""
    g = np.random.default_rng(11)
    W = g.integers(-8, 9, size=(12, 16)).astype(np.float64)
    got = oracle.block_norms(W, 4, kind)
    ex = _exact_block_sums(W, 4, kind)
    for r in range(3):
        for c in range(4):
            assert got[r, c] == float(ex[r][c])


@pytest.mark.parametrize("kind,b", [(1, 4), (2, 4), (1, 32), (2, 32)])
def test_norms_within_sum_error_bound(kind, b):
    """bf16 inputs of mixed magnitude: a left-to-right sum of n nonnegative terms has
    |computed - exact| <= (n - 1) u * exact, u = 2^-53 (textbook bound); the terms themselves
    are exact in fp64 (|w| of a bf16; w*w has 16 significant bits)."""
    W = synth.dense_weight(2 * b, 3 * b, seed=3, b=b).double().numpy()
    got = oracle.block_norms(W, b, kind)
    ex = _exact_block_sums(W, b, kind)
    n = b * b
    for r in range(2):
        for c in range(3):
            err = abs(Fraction(float(got[r, c])) - ex[r][c])
            assert err <= Fraction(n - 1, 2 ** 53) * ex[r][c]


def test_norm_closed_forms():
    b = 8
    W = np.zeros((2 * b, 2 * b))
    W[:b, :b] = -0.375                       # constant block: b^2 |c| and b^2 c^2
    W[b + 3, b + 5] = 2.5                    # a single nonzero
    n1, n2 = oracle.block_norms(W, b, 1), oracle.block_norms(W, b, 2)
    assert n1[0, 0] == b * b * 0.375 and n2[0, 0] == b * b * 0.375 ** 2
    assert n1[1, 1] == 2.5 and n2[1, 1] == 6.25
    assert n1[0, 1] == n1[1, 0] == 0 and n2[0, 1] == 0
    # scaling by a power of two scales every partial sum exactly
    Wr = synth.dense_weight(2 * b, 2 * b, seed=4).double().numpy()
    assert np.array_equal(oracle.block_norms(Wr * 8, b, 1), 8 * oracle.block_norms(Wr, b, 1))
    assert np.array_equal(oracle.block_norms(Wr * 8, b, 2), 64 * oracle.block_norms(Wr, b, 2))


@pytest.mark.parametrize("N,K,b", [(96, 64, 32), (128, 192, 64), (3072, 768, 32)])
def test_norms_match_reshape_reduction(N, K, b):
    """The same quantity by another formulation: reshape to [R, b, C, b] and reduce."""
    W = synth.dense_weight(N, K, seed=5, b=b).double().numpy()
    R, C = N // b, K // b
    for kind, t in ((1, np.abs(W)), (2, W * W)):
        alt = t.reshape(R, b, C, b).sum(axis=(1, 3))
        got = oracle.block_norms(W, b, kind)
        assert np.allclose(got, alt, rtol=1e-13, atol=0)


def test_topk_brute_force_over_subsets():
    """With distinct norms the kept set is the unique subset of size k with the largest
    total; every subset of a 2 x 4 grid is enumerated."""
    g = np.random.default_rng(7)
    for trial in range(6):
        norms = g.permutation(8).astype(np.float64).reshape(2, 4) + g.random() * 0.5
        for k in range(9):
            best = max(itertools.combinations(range(8), k), key=lambda s: sum(norms.ravel()[list(s)]))
            want = np.zeros(8, dtype=np.uint8)
            want[list(best)] = 1
            assert np.array_equal(convert.topk_mask(norms, k).ravel(), want), (trial, k)


def test_topk_ties_and_invariants():
    norms = np.array([[1.0, 3.0, 3.0], [2.0, 3.0, 0.0]])
    assert convert.topk_mask(norms, 2).tolist() == [[0, 1, 1], [0, 0, 0]]   # 3, 3 before the third 3
    assert convert.topk_mask(norms, 3).tolist() == [[0, 1, 1], [0, 1, 0]]
    assert convert.topk_mask(np.zeros((3, 3)), 4).ravel().tolist() == [1, 1, 1, 1, 0, 0, 0, 0, 0]
    g = np.random.default_rng(8)
    for _ in range(20):
        nrm = np.round(g.random((5, 7)) * 4) / 4          # many ties
        k = int(g.integers(0, 36))
        m = convert.topk_mask(nrm, k).ravel().astype(bool)
        assert m.sum() == k
        flat = nrm.ravel()
        if 0 < k < 35:
            assert flat[m].min() >= flat[~m].max()
            thr = flat[m].min()
            # among blocks equal to the threshold, the kept ones come first in index order
            tied = np.flatnonzero(flat == thr)
            kept = m[tied]
            assert not np.any(kept[1:] & ~kept[:-1])
    with pytest.raises(ValueError):
        convert.topk_mask(np.array([[np.nan, 1.0]]), 1)


@pytest.mark.parametrize("kind", [1, 2])
def test_selection_recovers_a_planted_support(kind):
    """A weight that is zero outside a block support: keeping exactly that many blocks
    returns the support."""
    N, K, b = 256, 384, 32
    mask = synth.uniform_mask(N // b, K // b, 0.3, np.random.default_rng(9))
    W = synth.dense_weight(N, K, seed=9).double().numpy()
    W[np.kron(mask, np.ones((b, b))) == 0] = 0.0
    got = convert.topk_mask(oracle.block_norms(W, b, kind), int(mask.sum()))
    assert np.array_equal(got, mask)


@pytest.mark.parametrize("N,K,b,d", [(256, 384, 32, 0.3), (512, 256, 64, 0.5), (96, 96, 32, 0.0), (64, 64, 32, 1.0)])
def test_round_trips_and_kron_mask(N, K, b, d):
    """values_to_dense(dense_to_values(W)) = W masked by kron(mask, ones(b, b)); the reverse
    is the identity on V. Raw bf16 bits are compared."""
    mask = synth.uniform_mask(N // b, K // b, d, np.random.default_rng(10))
    md = meta.scan(mask)
    W = synth.dense_weight(N, K, seed=10, b=b).view(torch.int16).numpy()
    V = convert.dense_to_values(W, md["row_ptr"], md["col_idx"], b)
    D = convert.values_to_dense(V, md["row_ptr"], md["col_idx"], N, K, b)
    assert np.array_equal(D, np.where(np.kron(mask, np.ones((b, b), dtype=np.uint8)) != 0, W, 0))
    assert np.array_equal(convert.dense_to_values(D, md["row_ptr"], md["col_idx"], b), V)


def test_bsr_from_dense_feeds_the_layer_contract():
    """The BSR values read out of a pruned dense weight, run through the oracle's forward,
    equal the dense product with that pruned weight (README workflow section)."""
    N, K, b, M = 256, 192, 32, 9
    W = synth.dense_weight(N, K, seed=12, b=b).double().numpy()
    mask = convert.topk_mask(oracle.block_norms(W, b, 1), 10)
    md = meta.scan(mask)
    V = convert.dense_to_values(W, md["row_ptr"], md["col_idx"], b)
    X = synth.activations(M, K, 12).double().numpy()
    Y, S = oracle.fwd(X, md["row_ptr"], md["col_idx"], V, N, b)
    Wp = np.where(np.kron(mask, np.ones((b, b))) != 0, W, 0.0)
    assert np.all(np.abs(Y - X @ Wp.T) <= 1e-12 * np.maximum(S, 1e-300))


def test_planted_mistakes_fail_a_pin():
    g = _golden()
    W = np.array(g["W"], dtype=np.float64)
    b, e = g["b"], g["bsr_l1_keep3"]
    md = dict(row_ptr=np.array(e["row_ptr"]), col_idx=np.array(e["col_idx"]))
    # a transposed block read
    Vt = convert.dense_to_values(W, md["row_ptr"], md["col_idx"], b).transpose(0, 2, 1)
    assert not np.array_equal(Vt, np.array(e["V"]))
    # ties to the higher index
    n1 = oracle.block_norms(W, b, 1).ravel()
    order = sorted(range(n1.size), key=lambda i: (-n1[i], -i))
    wrong = np.zeros(n1.size, np.uint8)
    wrong[order[:1]] = 1
    assert wrong.reshape(2, 3).tolist() != g["masks"][0]["mask"]
    # keeping the smallest norms instead of the largest
    small = np.zeros(n1.size, np.uint8)
    small[np.argsort(n1, kind="stable")[:3]] = 1
    assert small.reshape(2, 3).tolist() != g["masks"][2]["mask"]
    # norms stored column-major (an index slip in the [R][C] output)
    slip = oracle.block_norms(W, b, 1).ravel().reshape(3, 2).T
    assert not np.array_equal(slip, np.array(g["l1"]))
    # a dropped row term (the last row of every block not summed)
    n_drop = np.array([[np.abs(W[r * b:(r + 1) * b - 1, c * b:(c + 1) * b]).sum() for c in range(3)] for r in range(2)])
    assert not np.array_equal(n_drop, np.array(g["l1"]))
