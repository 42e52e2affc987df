"""The wide-tile panel GEMM (b = 32; forward and input gradient of dense groups, 256 x 256 tiles
with 4 x 4 accumulator grids per wave) against the fp64 oracle: full rows mixed with sparse and
empty ones, groups of fewer than 8 members, a last half panel, ragged row tiles, bias, integer
inputs (bit-exact), non-finite activations, bitwise determinism, and the automatic choice on the
Zipf 16384 x 4096 -> 11008 layer."""
import numpy as np
import pytest
import torch

import oracle
from oracle import meta
from sparse_gemm_amd import binding, synth
from sparse_gemm_amd.binding import Pattern

from gpu_util import case_inputs, check, dev, full_parity, say

pytestmark = pytest.mark.gpu


def mixed_mask(R, C, nfull, seed, empty_rows=(), density=0.15):
    """nfull random block rows kept in full, the others uniform at `density`, some rows empty."""
    g = np.random.default_rng(seed)
    mask = (g.random((R, C)) < density).astype(np.uint8)
    mask[g.choice(R, size=nfull, replace=False)] = 1
    for r in empty_rows:
        mask[r] = 0
    return mask


@pytest.mark.parametrize("M,R,C,nfull,seed", [
    (700, 20, 15, 10, 1),     # 3 groups (8, 8, 4 members), 15 block columns: a last half panel; 3 row tiles, ragged
    (256, 8, 16, 8, 2),       # one group, every row full: every sub-step dense
    (513, 33, 8, 20, 3),      # 5 groups, the last with one member; a one-row last tile
    (300, 24, 40, 3, 4),      # mostly sparse rows
])
def test_wide_matches_oracle(monkeypatch, M, R, C, nfull, seed):
    monkeypatch.setenv("BSR_GEMM_VARIANT", "4")
    b = 32
    mask = mixed_mask(R, C, nfull, seed, empty_rows=(R - 1,))
    say(f"case wide M={M} R={R} C={C} full={nfull} nnzb={int(mask.sum())}")
    host = case_inputs(M, R * b, C * b, b, seed, mask=mask, bias=True)
    full_parity(M, R * b, C * b, b, host, ops=("fwd", "dx"))


def test_wide_integer_inputs_bit_exact(monkeypatch):
    """Integer activations and blocks in {-2..2}: every product and fp32 sum is exact and |y| <= 256,
    so the wide kernels must equal the oracle bit for bit."""
    monkeypatch.setenv("BSR_GEMM_VARIANT", "4")
    M, R, C, b = 300, 16, 8, 32
    mask = mixed_mask(R, C, 9, 5)
    g = np.random.default_rng(5)
    nnzb = int(mask.sum())
    X = torch.from_numpy(g.integers(-2, 3, size=(M, C * b)).astype(np.float32)).to(torch.bfloat16)
    V = torch.from_numpy(g.integers(-1, 2, size=(nnzb, b, b)).astype(np.float32)).to(torch.bfloat16)
    dY = torch.from_numpy(g.integers(-1, 2, size=(M, R * b)).astype(np.float32)).to(torch.bfloat16)
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, R * b, C * b, b)
    Y = binding.linear_fwd(p, X.to(dev()), V.to(dev())).cpu()
    dX = binding.linear_bwd_input(p, dY.to(dev()), V.to(dev())).cpu()
    torch.cuda.synchronize()
    ref, _ = oracle.fwd(X, md["row_ptr"], md["col_idx"], V, R * b, b)
    assert np.array_equal(Y.double().numpy(), ref)
    ref, _ = oracle.dx(dY, md["row_ptr"], md["col_idx"], V, C * b, b)
    assert np.array_equal(dX.double().numpy(), ref)
    p.close()


def test_wide_nonfinite_activation_stays_in_its_blocks(monkeypatch):
    """An infinite activation reaches only the outputs of block rows that keep its input block,
    also inside dense sub-steps whose other members skip that block."""
    monkeypatch.setenv("BSR_GEMM_VARIANT", "4")
    M, R, C, b = 260, 16, 6, 32
    mask = np.ones((R, C), dtype=np.uint8)
    mask[1::3, 1] = 0
    mask[5, :] = 0
    mask[5, 1] = 1
    host = case_inputs(M, R * b, C * b, b, 23, mask=mask, bias=True)
    X = host["X"].clone()
    m_bad = 200
    X[m_bad, b + 9] = float("inf")
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, R * b, C * b, b)
    Y = binding.linear_fwd(p, X.to(dev()), host["V"].to(dev()), host["bias"].to(dev())).cpu()
    torch.cuda.synchronize()
    ref, S = oracle.fwd(host["X"], md["row_ptr"], md["col_idx"], host["V"], R * b, b, bias=host["bias"])
    uses = np.repeat(mask[:, 1].astype(bool), b)
    clean = np.ones((M, R * b), dtype=bool)
    clean[m_bad, uses] = False
    assert torch.isfinite(Y[~torch.from_numpy(clean)].float()).sum() == 0
    check("wide fwd (untouched)", Y[torch.from_numpy(clean)], ref[clean], S[clean])
    p.close()


def test_wide_is_deterministic(monkeypatch):
    monkeypatch.setenv("BSR_GEMM_VARIANT", "4")
    M, R, C, b = 1024, 24, 16, 32
    mask = mixed_mask(R, C, 12, 6)
    host = case_inputs(M, R * b, C * b, b, 6, mask=mask)
    p = Pattern.from_mask(mask, R * b, C * b, b)
    X, V, dY = host["X"].to(dev()), host["V"].to(dev()), host["dY"].to(dev())
    y1, y2 = binding.linear_fwd(p, X, V), binding.linear_fwd(p, X, V)
    d1, d2 = binding.linear_bwd_input(p, dY, V), binding.linear_bwd_input(p, dY, V)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))
    p.close()


# ---- the wide weight gradient (dense tiles of 4 full block rows x 16 consecutive block columns,
# then gathered tiles of any 4 rows x any 16 columns taking every other block, whose sparser tiles
# give their blocks to thin items of 8 single blocks, one wave each: every case below but the two
# all-dense ones has thin items, some with fewer than 8 blocks, and M = 1000 splits them over row
# chunks) ----

@pytest.mark.parametrize("M,R,C,nfull,seed", [
    (300, 21, 40, 9, 7),      # 21 rows: 2 dense row groups, 8 leftover columns, gathered rows
    (1000, 12, 32, 8, 8),     # gathered items split over row chunks (fp32 partials + reduce); M ragged
    (4133, 16, 16, 16, 9),    # every block kept: every tile dense
    (97, 9, 24, 5, 10),       # M below one 32-row step past 64, ragged steps
    (1, 8, 16, 8, 11),        # one activation row: 31 rows of each step read as zeros
    (45, 10, 20, 6, 12),      # 45 rows, 20 columns (a partial 16-column gather)
])
def test_wide_dw_matches_oracle(M, R, C, nfull, seed):
    b = 32
    mask = mixed_mask(R, C, nfull, seed, empty_rows=(R - 1,) if nfull < R else ())
    say(f"case wide dW M={M} R={R} C={C} full={nfull} nnzb={int(mask.sum())}")
    host = case_inputs(M, R * b, C * b, b, seed, mask=mask, bias=True)
    full_parity(M, R * b, C * b, b, host, ops=("dw",), dbias=True)


def test_wide_dw_integer_inputs_bit_exact():
    """Small-integer activations and gradients: every fp32 sum over the rows is exact, so dV equals
    the oracle bit for bit, through both the dense and the gathered wide tiles."""
    M, R, C, b = 700, 10, 32, 32
    mask = mixed_mask(R, C, 6, 11)
    g = np.random.default_rng(11)
    X = torch.from_numpy(g.integers(-2, 3, size=(M, C * b)).astype(np.float32)).to(torch.bfloat16)
    dY = torch.from_numpy(g.integers(-1, 2, size=(M, R * b)).astype(np.float32)).to(torch.bfloat16)
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, R * b, C * b, b)
    dV, _ = binding.linear_bwd_weight(p, dY.to(dev()), X.to(dev()))
    torch.cuda.synchronize()
    ref, _ = oracle.dw(dY, X, md["row_ptr"], md["col_idx"], b)
    assert np.array_equal(dV.cpu().double().numpy(), ref)
    p.close()


def test_wide_dw_is_deterministic():
    M, R, C, b = 2048, 16, 32, 32
    mask = mixed_mask(R, C, 10, 12)
    host = case_inputs(M, R * b, C * b, b, 12, mask=mask)
    p = Pattern.from_mask(mask, R * b, C * b, b)
    X, dY = host["X"].to(dev()), host["dY"].to(dev())
    a1, _ = binding.linear_bwd_weight(p, dY, X)
    a2, _ = binding.linear_bwd_weight(p, dY, X)
    torch.cuda.synchronize()
    assert torch.equal(a1.view(torch.int16), a2.view(torch.int16))
    p.close()
