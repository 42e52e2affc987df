"""Seeded input generators and the oracle's metadata scan (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import meta
from sparse_gemm_amd import synth


def test_seed_determinism():
    w = synth.WORKLOADS[2].with_m(64)
    a = synth.make_inputs(w, seed=3)
    b = synth.make_inputs(w, seed=3)
    c = synth.make_inputs(w, seed=4)
    assert np.array_equal(a["mask"], b["mask"])
    for k in ("X", "V", "dY"):
        assert torch.equal(a[k], b[k])
    assert not np.array_equal(a["mask"], c["mask"])


def test_row_prefix_independent_of_m():
    x_small = synth.activations(16, 256, 7)
    x_big = synth.activations(64, 256, 7)
    assert torch.equal(x_small, x_big[:16])


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_uniform_counts(k):
    w = synth.WORKLOADS[k]
    mask = synth.block_mask(w, 0)
    assert mask.shape == (w.R, w.C)
    assert int(mask.sum()) == int(np.floor(w.density * w.R * w.C + 0.5))
    assert set(np.unique(mask)) <= {0, 1}


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_zipf_counts(seed):
    w = synth.WORKLOADS[5]
    mask = synth.block_mask(w, seed)
    counts = mask.sum(axis=1)
    assert int(counts.sum()) == round(0.3 * w.R * w.C) == 13210
    assert counts.min() >= 1 and counts.max() <= w.C
    h = synth.row_histogram(mask)
    assert 80 <= h["full_rows"] <= 100 and 190 <= h["single_rows"] <= 215


def test_value_distributions():
    V = synth.block_values(200, 32, 0).float()
    assert abs(V.std().item() - 0.02) < 0.001 and abs(V.mean().item()) < 0.001
    X = synth.activations(256, 256, 0).float()
    assert abs(X.std().item() - 1.0) < 0.02
    assert X.dtype == torch.float32 and synth.activations(2, 2, 0).dtype == torch.bfloat16


def test_bf16_rounding_is_rne():
    # 1 + 2^-8 lies exactly between bf16 neighbours 1 and 1 + 2^-7: ties go to even (1.0)
    t = synth.to_bf16(np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32)).float()
    assert t.tolist() == [1.0, 1.0 + 2.0 ** -6]


def _check_invariants(mask, md):
    R, C = mask.shape
    rp, ci, cp, ri, pm = (md[k] for k in ("row_ptr", "col_idx", "col_ptr", "row_idx", "perm"))
    nnzb = int(mask.sum())
    assert rp[0] == 0 and rp[-1] == nnzb and np.all(np.diff(rp) >= 0) and len(rp) == R + 1
    assert cp[0] == 0 and cp[-1] == nnzb and np.all(np.diff(cp) >= 0) and len(cp) == C + 1
    for r in range(R):
        cols = ci[rp[r]:rp[r + 1]]
        assert np.all(np.diff(cols) > 0)
        assert sorted(np.nonzero(mask[r])[0].tolist()) == cols.tolist()
    assert sorted(pm.tolist()) == list(range(nnzb))
    row_of = np.repeat(np.arange(R), np.diff(rp))
    for c in range(C):
        rows = ri[cp[c]:cp[c + 1]]
        assert np.all(np.diff(rows) > 0)
        for j in range(cp[c], cp[c + 1]):
            assert row_of[pm[j]] == ri[j] and ci[pm[j]] == c


@pytest.mark.parametrize("R,C,d,seed", [(1, 1, 1.0, 0), (7, 5, 0.3, 1), (16, 40, 0.1, 2), (40, 16, 0.9, 3),
                                        (9, 9, 0.0, 4)])
def test_meta_invariants(R, C, d, seed):
    mask = synth.uniform_mask(R, C, d, np.random.default_rng(seed))
    _check_invariants(mask, meta.scan(mask))


def test_meta_invariants_zipf():
    mask = synth.block_mask(synth.WORKLOADS[5], 0)
    _check_invariants(mask, meta.scan(mask))
