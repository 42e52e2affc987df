"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by element.

Acceptance: |g - ref| <= 4e-3 * S per element (S = sum of |products|, bf16 inputs and
outputs, fp32 accumulation), g == ref where S == 0; metadata and integer-valued cases are
bit-exact. The five reference workloads run at full size: fully checked where the oracle is
cheap, otherwise on sampled rows (forward, input gradient) and sampled blocks over the full
M (weight gradient).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import meta
from sparse_gemm_amd import binding, synth
from sparse_gemm_amd.binding import Pattern

from gpu_util import case_inputs, check, dev, full_parity, say, to_dev

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ small and ragged shapes

@pytest.mark.parametrize("M,N,K,b,d,seed", [
    (1, 256, 256, 32, 0.5, 0),
    (7, 512, 256, 32, 0.4, 1),
    (8, 256, 512, 64, 0.5, 2),
    (15, 384, 192, 32, 0.3, 3),
    (16, 256, 256, 64, 0.5, 4),
    (17, 256, 256, 32, 0.5, 5),
    (100, 320, 448, 32, 0.35, 6),
    (257, 512, 384, 64, 0.4, 7),
    (300, 256, 1024, 32, 0.2, 8),
    (513, 1024, 512, 32, 0.15, 9),
    (129, 512, 512, 64, 1.0, 10),
])
def test_shapes(M, N, K, b, d, seed):
    say(f"case shapes M={M} N={N} K={K} b={b} d={d} seed={seed}")
    host = case_inputs(M, N, K, b, seed, density=d, bias=True)
    full_parity(M, N, K, b, host, dbias=True)


@pytest.mark.parametrize("M,N,K,b,d,seed", [
    (300, 96, 256, 32, 0.5, 14),    # 96 columns: a 64-column group of the bias sums is half outside
    (1000, 160, 128, 32, 0.5, 15),  # 3 row chunks of 334 rows (not a multiple of the 32 row lanes)
    (5000, 224, 64, 32, 0.6, 16),   # 19 chunks of 264 rows: a second, partial batch of 8 rows per lane
    (33, 192, 128, 64, 0.5, 17),
])
def test_bias_gradient_ragged(M, N, K, b, d, seed):
    """The bias gradient's column sums over ragged row chunks and column groups, with the rest of
    the step."""
    say(f"case bias gradient M={M} N={N} K={K} b={b} d={d}")
    host = case_inputs(M, N, K, b, seed, density=d, bias=True)
    full_parity(M, N, K, b, host, dbias=True)


@pytest.mark.parametrize("variant", ["0", "1", "2", "3", "4"])
@pytest.mark.parametrize("M,N,K,b,seed", [
    (300, 512, 480, 32, 11),   # 15 block columns: the last 64-column panel is half a panel
    (300, 512, 448, 64, 12),
    (260, 768, 256, 32, 13),   # dense enough that panels fill every slot
])
def test_every_gemm_variant(monkeypatch, variant, M, N, K, b, seed):
    """Every forward / input-gradient kernel variant (256-row work-groups with 8 slots, 128-row
    with 4, 128-row with half-width and single-member groups), whichever the automatic choice would take for this
    size, over a ragged row tail."""
    monkeypatch.setenv("BSR_GEMM_VARIANT", variant)
    say(f"case variant={variant} M={M} N={N} K={K} b={b} seed={seed}")
    host = case_inputs(M, N, K, b, seed, density=0.4 if seed != 13 else 0.8, bias=True)
    full_parity(M, N, K, b, host, dbias=True)


@pytest.mark.parametrize("b,M,bad_rows", [(64, 24, (20,)), (64, 57, (40, 56)), (32, 24, (17, 23))])
def test_nonfinite_activation_small_m_tiles(b, M, bad_rows):
    """The small-M forward with 2 or 4 activation tiles of 16 rows per work-group: an infinite
    activation in a row of tile 1, 2 or 3 reaches only that row's outputs of block rows that keep
    its input block. Rows of other tiles, and block rows whose passes run past their last kept
    block (those blocks read zeros for both operands), stay finite and match the oracle."""
    R, C = 6, 4
    mask = np.ones((R, C), dtype=np.uint8)
    mask[0::2, 1] = 0             # even block rows skip input block 1
    mask[3, 2:] = 0               # block row 3 ends early
    mask[5, :] = 0
    mask[5, 1] = 1                # block row 5 keeps only block 1
    host = case_inputs(M, R * b, C * b, b, 22, mask=mask, bias=True, dy=False)
    say(f"case non-finite activation small-M b={b} M={M} rows={bad_rows}")
    X = host["X"].clone()
    for m in bad_rows:
        X[m, b + 7] = float("inf")   # input block 1
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, R * b, C * b, b)
    Y = binding.linear_fwd(p, X.to(dev()), host["V"].to(dev()), host["bias"].to(dev())).cpu()
    torch.cuda.synchronize()
    ref, S = oracle.fwd(host["X"], md["row_ptr"], md["col_idx"], host["V"], R * b, b, bias=host["bias"])
    uses = np.repeat(mask[:, 1].astype(bool), b)
    clean = np.ones((M, R * b), dtype=bool)
    for m in bad_rows:
        clean[m, uses] = False
    assert torch.isfinite(Y[~torch.from_numpy(clean)].float()).sum() == 0
    check("fwd small-M tiles (untouched)", Y[torch.from_numpy(clean)], ref[clean], S[clean])
    p.close()


@pytest.mark.parametrize("variant", ["0", "1", "2", "3", "4"])
@pytest.mark.parametrize("M", [9, 300])
def test_nonfinite_activation_stays_in_its_blocks(monkeypatch, variant, M):
    """The layer sums over kept blocks only: an infinite activation in input block 1 reaches the
    outputs of block rows that keep a block in column 1 and no others, also where another member
    of the same 64-column panel group skips block 1 (a skipped block must not be multiplied as a
    zero block: zero times infinity is NaN). Same for an infinite output gradient and the input
    gradient. M = 9 takes the small-M forward."""
    monkeypatch.setenv("BSR_GEMM_VARIANT", variant)
    b, R, C = 32, 8, 4
    mask = np.ones((R, C), dtype=np.uint8)
    mask[0::2, 1] = 0             # even block rows skip input block 1 ...
    mask[:, 3] = 0
    mask[5, :] = 0
    mask[5, 1] = 1                # ... and block row 5 keeps only block 1
    host = case_inputs(M, R * b, C * b, b, 21, mask=mask, bias=True)
    say(f"case non-finite activation variant={variant} M={M}")
    m_bad = M // 2
    X, dY = host["X"].clone(), host["dY"].clone()
    X[m_bad, b + 3] = float("inf")
    dY[m_bad, 2 * b + 5] = float("-inf")   # block row 2 (keeps input blocks 0 and 2)
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, R * b, C * b, b)
    Y = binding.linear_fwd(p, X.to(dev()), host["V"].to(dev()), host["bias"].to(dev())).cpu()
    dX = binding.linear_bwd_input(p, dY.to(dev()), host["V"].to(dev())).cpu()
    torch.cuda.synchronize()
    # outputs that do not touch the infinite entry match the oracle on the finite inputs
    ref, S = oracle.fwd(host["X"], md["row_ptr"], md["col_idx"], host["V"], R * b, b, bias=host["bias"])
    uses = np.repeat(mask[:, 1].astype(bool), b)            # output columns whose block row keeps block 1
    clean = np.ones((M, R * b), dtype=bool)
    clean[m_bad, uses] = False
    assert torch.isfinite(Y[~torch.from_numpy(clean)].float()).sum() == 0
    check("fwd (untouched)", Y[torch.from_numpy(clean)], ref[clean], S[clean])
    ref, S = oracle.dx(host["dY"], md["row_ptr"], md["col_idx"], host["V"], C * b, b)
    uses = np.repeat(mask[2, :].astype(bool), b)            # input columns fed by block row 2
    clean = np.ones((M, C * b), dtype=bool)
    clean[m_bad, uses] = False
    assert torch.isfinite(dX[~torch.from_numpy(clean)].float()).sum() == 0
    check("dx (untouched)", dX[torch.from_numpy(clean)], ref[clean], S[clean])
    p.close()


@pytest.mark.parametrize("b", [32, 64])
def test_empty_rows_and_columns(b):
    R, C = 6, 5
    mask = np.zeros((R, C), dtype=np.uint8)
    mask[0, 1] = mask[0, 3] = mask[2, 1] = mask[5, 4] = mask[5, 0] = 1   # rows 1, 3, 4 and column 2 empty
    for M in (5, 70):
        say(f"case empty rows/cols b={b} M={M}")
        host = case_inputs(M, R * b, C * b, b, 11, mask=mask, bias=True)
        full_parity(M, R * b, C * b, b, host, dbias=True)


@pytest.mark.parametrize("b", [32, 64])
def test_no_blocks(b):
    mask = np.zeros((3, 4), dtype=np.uint8)
    say(f"case nnzb=0 b={b}")
    host = case_inputs(33, 3 * b, 4 * b, b, 12, mask=mask, bias=True)
    full_parity(33, 3 * b, 4 * b, b, host, dbias=True)


def test_m_zero():
    say("case M=0")
    b = 32
    mask = np.ones((2, 2), dtype=np.uint8)
    p = Pattern.from_mask(mask, 64, 64, b)
    V = synth.block_values(4, b, 0).to(dev())
    X = torch.empty((0, 64), dtype=torch.bfloat16, device=dev())
    Y = binding.linear_fwd(p, X, V)
    dX = binding.linear_bwd_input(p, torch.empty((0, 64), dtype=torch.bfloat16, device=dev()), V)
    dV, db = binding.linear_bwd_weight(p, torch.empty((0, 64), dtype=torch.bfloat16, device=dev()), X,
                                       want_dbias=True,
                                       out=torch.full((4, b, b), float("nan"), dtype=torch.bfloat16, device=dev()),
                                       dbias=torch.full((64,), float("nan"), dtype=torch.bfloat16, device=dev()))
    torch.cuda.synchronize()
    assert Y.shape == (0, 64) and dX.shape == (0, 64)
    assert torch.all(dV == 0) and torch.all(db == 0)


# ------------------------------------------------------------------ exact cases

@pytest.mark.parametrize("b", [32, 64])
def test_integer_inputs_bit_exact(b):
    """Entries in {-1, 0, 1} with at most 256 products per output: every fp32 sum is exact and
    bf16 holds integers up to 256, so the GPU must match the oracle bit for bit."""
    N = K = 256
    M = 200
    g = np.random.default_rng(5)
    mask = (g.random((N // b, K // b)) < 0.6).astype(np.uint8)
    md = meta.scan(mask)
    X = torch.from_numpy(g.integers(-1, 2, size=(M, K)).astype(np.float32)).to(torch.bfloat16)
    V = torch.from_numpy(g.integers(-1, 2, size=(md["nnzb"], b, b)).astype(np.float32)).to(torch.bfloat16)
    dY = torch.from_numpy(g.integers(-1, 2, size=(M, N)).astype(np.float32)).to(torch.bfloat16)
    say(f"case integer exact b={b}")
    p = Pattern.from_mask(mask, N, K, b)
    Xd, Vd, dYd = X.to(dev()), V.to(dev()), dY.to(dev())
    Y = binding.linear_fwd(p, Xd, Vd)
    dX = binding.linear_bwd_input(p, dYd, Vd)
    dV, db = binding.linear_bwd_weight(p, dYd, Xd, want_dbias=True)
    torch.cuda.synchronize()
    Yr, _ = oracle.fwd(X, md["row_ptr"], md["col_idx"], V, N, b)
    dXr, _ = oracle.dx(dY, md["row_ptr"], md["col_idx"], V, K, b)
    dVr, _ = oracle.dw(dY, X, md["row_ptr"], md["col_idx"], b)
    dbr, _ = oracle.db(dY)
    assert np.array_equal(Y.cpu().double().numpy(), Yr)
    assert np.array_equal(dX.cpu().double().numpy(), dXr)
    assert np.array_equal(dV.cpu().double().numpy(), dVr)
    assert np.array_equal(db.cpu().double().numpy(), dbr)


@pytest.mark.parametrize("b", [32, 64])
def test_permutation_blocks_bit_exact(b):
    R = 5
    sigma = [2, 4, 0, 3, 1]
    mask = np.zeros((R, R), dtype=np.uint8)
    for r in range(R):
        mask[r, sigma[r]] = 1
    V = torch.stack([torch.eye(b)] * R).to(torch.bfloat16)
    X = synth.activations(77, R * b, 1)
    say(f"case permutation b={b}")
    p = Pattern.from_mask(mask, R * b, R * b, b)
    Y = binding.linear_fwd(p, X.to(dev()), V.to(dev())).cpu()
    dX = binding.linear_bwd_input(p, X.to(dev()), V.to(dev())).cpu()
    for r in range(R):
        assert torch.equal(Y[:, r * b:(r + 1) * b], X[:, sigma[r] * b:(sigma[r] + 1) * b])
        assert torch.equal(dX[:, sigma[r] * b:(sigma[r] + 1) * b], X[:, r * b:(r + 1) * b])


# ------------------------------------------------------------------ coverage and determinism

@pytest.mark.parametrize("b,M", [(32, 9), (32, 300), (64, 12), (64, 190)])
def test_nan_poisoned_outputs_are_overwritten(b, M):
    N, K = 8 * b, 6 * b
    mask = synth.uniform_mask(8, 6, 0.3, np.random.default_rng(3))
    mask[2, :] = 0
    mask[:, 4] = 0
    host = to_dev(case_inputs(M, N, K, b, 3, mask=mask, bias=True))
    say(f"case nan poison b={b} M={M}")
    p = Pattern.from_mask(mask, N, K, b)
    nan = lambda *s: torch.full(s, float("nan"), dtype=torch.bfloat16, device=dev())
    Y = binding.linear_fwd(p, host["X"], host["V"], host["bias"], out=nan(M, N))
    dX = binding.linear_bwd_input(p, host["dY"], host["V"], out=nan(M, K))
    dV, db = binding.linear_bwd_weight(p, host["dY"], host["X"], out=nan(p.nnzb, b, b), dbias=nan(N))
    torch.cuda.synchronize()
    for t in (Y, dX, dV, db):
        assert torch.isfinite(t.float()).all()


def test_runs_are_bitwise_deterministic():
    w = synth.WORKLOADS[2]
    host = to_dev(synth.make_inputs(w, 0))
    say("case determinism (BERT-base FFN-up shape)")
    p = Pattern.from_mask(host["mask"], w.N, w.K, w.b)
    outs = []
    for _ in range(2):
        Y = binding.linear_fwd(p, host["X"], host["V"])
        dX = binding.linear_bwd_input(p, host["dY"], host["V"])
        dV, db = binding.linear_bwd_weight(p, host["dY"], host["X"], want_dbias=True)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (Y, dX, dV, db)])
    for a, c in zip(*outs):
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))


# ------------------------------------------------------------------ error codes on the device path

def test_error_codes():
    import ctypes
    from sparse_gemm_amd import _lib
    L = _lib.load()
    b = 32
    mask = np.ones((2, 2), dtype=np.uint8)
    p = Pattern.from_mask(mask, 64, 64, b)
    X = torch.zeros((8, 65), dtype=torch.bfloat16, device=dev())
    V = torch.zeros((4, b, b), dtype=torch.bfloat16, device=dev())
    Y = torch.zeros((8, 64), dtype=torch.bfloat16, device=dev())
    mis = ctypes.c_void_p(X.data_ptr() + 2)          # one element off: not 16-byte aligned
    ok = ctypes.c_void_p(X.data_ptr())
    vp, yp = ctypes.c_void_p(V.data_ptr()), ctypes.c_void_p(Y.data_ptr())
    assert L.bsr_linear_fwd(p.handle, mis, 8, vp, None, yp, None) == 3
    assert L.bsr_linear_fwd(p.handle, ok, -1, vp, None, yp, None) == 1
    assert L.bsr_linear_fwd(p.handle, None, 8, vp, None, yp, None) == 1
    need = L.bsr_linear_bwd_weight_workspace(p.handle, 4096)
    big = torch.zeros((4096, 64), dtype=torch.bfloat16, device=dev())
    bp = ctypes.c_void_p(big.data_ptr())
    if need:
        ws = torch.zeros((need,), dtype=torch.uint8, device=dev())
        assert L.bsr_linear_bwd_weight(p.handle, bp, bp, 4096, vp, None, ctypes.c_void_p(ws.data_ptr()), need - 1,
                                       None) == 4
    torch.cuda.synchronize()
    assert torch.all(Y == 0) and torch.all(V == 0)   # nothing written on error


# ------------------------------------------------------------------ the reference workloads

def _sampled_parity(w: synth.Workload, seed: int, nrows: int, nblocks: int):
    host = synth.make_inputs(w, seed)
    d = to_dev(host)
    md = meta.scan(host["mask"])
    p = Pattern.from_mask(host["mask"], w.N, w.K, w.b)
    g = np.random.default_rng([seed, 77])
    rows = np.unique(np.concatenate([[0, w.M - 1], g.choice(w.M, size=min(nrows, w.M), replace=False)]))
    rows_t = torch.from_numpy(rows)
    if "fwd" in w.ops:
        Y = binding.linear_fwd(p, d["X"], d["V"], d["bias"])
        torch.cuda.synchronize()
        ref, S = oracle.fwd(host["X"][rows_t], md["row_ptr"], md["col_idx"], host["V"], w.N, w.b, bias=host["bias"])
        check(f"fwd ({rows.size} sampled rows)", Y.cpu()[rows_t], ref, S)
        del Y
    if "dx" in w.ops:
        dX = binding.linear_bwd_input(p, d["dY"], d["V"])
        torch.cuda.synchronize()
        ref, S = oracle.dx(host["dY"][rows_t], md["row_ptr"], md["col_idx"], host["V"], w.K, w.b)
        check(f"dx ({rows.size} sampled rows)", dX.cpu()[rows_t], ref, S)
        del dX
    if "dw" in w.ops:
        dV, _ = binding.linear_bwd_weight(p, d["dY"], d["X"])
        torch.cuda.synchronize()
        counts = np.diff(md["row_ptr"])
        row_of = np.repeat(np.arange(w.R), counts)
        # blocks from the fullest and the emptiest rows, plus a uniform sample, plus first/last
        heavy = np.nonzero(counts[row_of] == counts.max())[0]
        light = np.nonzero(counts[row_of] == counts[counts > 0].min())[0]
        pick = [0, md["nnzb"] - 1] + list(g.choice(heavy, size=min(8, heavy.size), replace=False)) + \
            list(g.choice(light, size=min(8, light.size), replace=False)) + \
            list(g.choice(md["nnzb"], size=min(nblocks, md["nnzb"]), replace=False))
        blocks = np.unique(np.asarray(pick, dtype=np.int64))
        ref, S = oracle.dw(host["dY"], host["X"], md["row_ptr"], md["col_idx"], w.b, blocks=blocks)
        check(f"dw ({blocks.size} sampled blocks, full M)", dV.cpu()[torch.from_numpy(blocks)], ref, S)
    p.close()


@pytest.mark.parametrize("k", [1, 2, 4])
def test_workload_full(k):
    w = synth.WORKLOADS[k]
    say(f"case workload {w.name} (full oracle)")
    host = synth.make_inputs(w, 0)
    full_parity(w.M, w.N, w.K, w.b, host, ops=w.ops)


@pytest.mark.parametrize("k,nrows,nblocks", [(3, 160, 32), (5, 96, 24)])
def test_workload_sampled(k, nrows, nblocks):
    w = synth.WORKLOADS[k]
    say(f"case workload {w.name} (sampled oracle)")
    _sampled_parity(w, 0, nrows, nblocks)


@pytest.mark.parametrize("cfg", ["0", "1", "2", "3", "4", "5", "6", "7"])
@pytest.mark.parametrize("M,N,K,b,d,seed", [(8, 512, 512, 64, 0.5, 90), (16, 384, 640, 64, 0.45, 91),
                                            (3, 256, 512, 32, 0.4, 92), (13, 640, 320, 32, 0.6, 93),
                                            (29, 512, 512, 64, 0.5, 96), (32, 384, 256, 32, 0.5, 97)])
def test_every_small_m_config(monkeypatch, cfg, M, N, K, b, d, seed):
    """Every small-M forward configuration (waves, blocks per pass, slices per work-group, loads of
    the next pass overlapped or not), whichever the default is, with bias and rows past M."""
    monkeypatch.setenv("BSR_SMALLM_CONFIG", cfg)
    say(f"case small-M config={cfg} M={M} N={N} K={K} b={b} d={d}")
    host = case_inputs(M, N, K, b, seed, density=d, bias=True, dy=False)
    full_parity(M, N, K, b, host, ops=("fwd",))


@pytest.mark.parametrize("limit,M,N,K,b,d,seed", [
    ("", 17, 512, 512, 64, 0.5, 100), ("", 32, 512, 384, 32, 0.45, 101), ("", 25, 3584, 1024, 64, 0.5, 102),
    ("", 57, 512, 512, 64, 0.5, 106), ("", 64, 896, 640, 64, 0.4, 107),
    ("80", 48, 384, 512, 64, 0.5, 103), ("80", 80, 640, 320, 32, 0.4, 104), ("80", 71, 256, 256, 32, 0.6, 105),
])
@pytest.mark.parametrize("cfg", ["", "6"])
def test_small_m_row_chunks(monkeypatch, cfg, limit, M, N, K, b, d, seed):
    """The small-M forward with 2 or 4 activation tiles of 16 rows per work-group and several grid rows,
    a ragged last tile and bias: by default up to 64 rows (b = 64) or 32 (b = 32), and up to 80 rows
    with the dispatch limit raised."""
    if limit:
        monkeypatch.setenv("BSR_SMALLM_MAX", limit)
    if cfg:
        monkeypatch.setenv("BSR_SMALLM_CONFIG", cfg)
    say(f"case small-M row chunks cfg={cfg or 'default'} limit={limit or 'default'} M={M} N={N} K={K} b={b} d={d}")
    host = case_inputs(M, N, K, b, seed, density=d, bias=True, dy=False)
    full_parity(M, N, K, b, host, ops=("fwd",))
