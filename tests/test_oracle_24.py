"""Pins of the oracle's 2:4 sparsity inside kept blocks, from facts outside the oracle:
  * a hand-worked block (tests/golden/sparse24_b16.json);
  * brute force over the six position pairs of every group: the kept pair has the largest sum of
    magnitudes, the lexicographically smallest such pair (the page's "remove the lowest norm"
    rule with ties to the lower position);
  * blocks that already are 2:4 with distinct magnitudes pass through unchanged;
  * kept magnitudes dominate dropped ones in every group;
  * the forward with the decompressed blocks equals the dense product with the pruned weight;
  * planted mistakes (keeping the smallest, swapped index fields) fail a pin.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle import meta
from sparse_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PAIRS = list(itertools.combinations(range(4), 2))


def _brute_pair(g):
    best = max(abs(g[a]) + abs(g[b]) for a, b in PAIRS)
    return min((a, b) for a, b in PAIRS if abs(g[a]) + abs(g[b]) == best)


def test_golden_block():
    fx = json.load(open(os.path.join(GOLDEN, "sparse24_b16.json")))
    V = np.array(fx["V"], dtype=np.float64)
    Vc, mt = oracle.compress_24(V)
    assert np.array_equal(Vc, np.array(fx["Vc"]))
    assert np.array_equal(mt, np.array(fx["meta"], dtype=np.uint16))
    assert np.array_equal(oracle.decompress_24(Vc, mt), np.array(fx["dense"]))


def test_every_small_group_against_brute_force():
    """All groups with magnitudes in {0, 1, 2} and both signs (many ties)."""
    groups = [np.array(m) * np.array(s) for m in itertools.product([0, 1, 2], repeat=4)
              for s in ([1, 1, 1, 1], [-1, 1, -1, 1])]
    b = 16
    rows = len(groups) // (b // 4) + 1
    flat = np.zeros((rows * b // 4, 4))
    flat[:len(groups)] = np.array(groups)
    nblk = -(-rows // b)
    V = np.zeros((nblk * b * (b // 4), 4))
    V[:flat.shape[0]] = flat
    V = V.reshape(nblk, b, b)
    Vc, mt = oracle.compress_24(V)
    D = oracle.decompress_24(Vc, mt)
    for i in range(nblk):
        for p in range(b):
            for h in range(b // 4):
                g = V[i, p, 4 * h:4 * h + 4]
                a, c = _brute_pair(g)
                want = np.zeros(4)
                want[a], want[c] = g[a], g[c]
                assert np.array_equal(D[i, p, 4 * h:4 * h + 4], want), (g, D[i, p, 4 * h:4 * h + 4])
                bits = (int(mt[i, p, h // 4]) >> (4 * (h % 4))) & 15
                assert (bits & 3, bits >> 2) == (a, c)
                assert np.array_equal(Vc[i, p, 2 * h:2 * h + 2], [g[a], g[c]])


@pytest.mark.parametrize("b", [16, 32, 64])
def test_random_blocks_dominance_and_half_density(b):
    V = synth.block_values(20, b, seed=b).double().numpy()
    Vc, mt = oracle.compress_24(V)
    D = oracle.decompress_24(Vc, mt)
    G = V.reshape(20, b, b // 4, 4)
    K = D.reshape(20, b, b // 4, 4)
    kept = K != 0
    assert np.all(kept.sum(axis=3) == 2)          # N(0, 0.02) draws: no zeros, so exactly 2 kept
    assert np.array_equal(K[kept], G[kept])
    mag = np.abs(G)
    assert np.all(np.where(kept, mag, np.inf).min(axis=3) >= np.where(~kept, mag, -np.inf).max(axis=3))


def test_already_24_blocks_pass_through():
    g = np.random.default_rng(3)
    b, n = 32, 6
    V = np.zeros((n, b, b))
    for i in range(n):
        for p in range(b):
            for h in range(b // 4):
                a, c = PAIRS[g.integers(6)]
                V[i, p, 4 * h + a] = g.choice([-1, 1]) * (1 + g.integers(1, 100)) / 64
                V[i, p, 4 * h + c] = g.choice([-1, 1]) * (101 + g.integers(1, 100)) / 64
    Vc, mt = oracle.compress_24(V)
    assert np.array_equal(oracle.decompress_24(Vc, mt), V)


def test_forward_contract_with_pruned_blocks():
    N, K, b, M = 256, 192, 32, 7
    mask = synth.uniform_mask(N // b, K // b, 0.5, np.random.default_rng(4))
    md = meta.scan(mask)
    V = synth.block_values(int(mask.sum()), b, 4)
    D = oracle.decompress_24(*oracle.compress_24(V))
    X = synth.activations(M, K, 4)
    Y, S = oracle.fwd(X, md["row_ptr"], md["col_idx"], D, N, b)
    W = meta.dense_weight(md["row_ptr"], md["col_idx"], D, N, K, b)
    assert np.all(np.abs(Y - X.double().numpy() @ W.T) <= 1e-12 * np.maximum(S, 1e-300))
    assert np.count_nonzero(W) * 2 == np.count_nonzero(meta.dense_weight(md["row_ptr"], md["col_idx"],
                                                                        V.double().numpy(), N, K, b))


def test_planted_mistakes_fail_a_pin():
    g = np.array([3.0, -1.0, 0.5, 2.0])
    # keeping the two smallest magnitudes
    small = tuple(sorted(np.argsort(np.abs(g), kind="stable")[:2]))
    assert small != _brute_pair(g)
    # the two index fields swapped inside a group's nibble
    fx = json.load(open(os.path.join(GOLDEN, "sparse24_b16.json")))
    _, mt = oracle.compress_24(np.array(fx["V"], dtype=np.float64))
    swapped = ((mt & 0x3333) << 2) | ((mt >> 2) & 0x3333)
    assert not np.array_equal(swapped, np.array(fx["meta"], dtype=np.uint16))
