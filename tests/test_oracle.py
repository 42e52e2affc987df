"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each pin is fixed by the pages or by the mathematics, not by re-typing the
oracle's loops:
  * hand-worked example (tests/golden/worked_example_b2.json);
  * the dense masked GEMM: block-sparse results equal dense matmul with zeros
    in the missing places (pytorch/ao sparsity README, workflow section), and
    the weight gradient is the dense gradient masked to the pattern (README,
    out-of-place update dW' = dW (Mask));
  * exact Fraction brute force over the scalar definition on tiny inputs;
  * adjoint identities <Y - b, dY> = <X, dX> = sum_i <dV_i, V_i>;
  * closed forms: identity / permutation blocks, a single dense block (a plain
    GEMM), M = 1 (a GEMV);
  * planted mistakes (a transposed block, a dropped bias, a shifted column
    index, a dropped block) must each fail at least one pin.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import brute, meta
from sparse_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(M, N, K, b, density, seed, bias=True, mask=None):
    R, C = N // b, K // b
    g = synth.rng(seed, synth.STREAM_PATTERN)
    if mask is None:
        mask = synth.uniform_mask(R, C, density, g)
    nnzb = int(mask.sum())
    X = synth.activations(M, K, seed)
    V = synth.block_values(nnzb, b, seed)
    bb = synth.bias_vector(N, seed) if bias else None
    dY = synth.grad_output(M, N, seed)
    md = meta.scan(mask)
    return dict(mask=mask, X=X, V=V, bias=bb, dY=dY, md=md, M=M, N=N, K=K, b=b)


def _dense_refs(c):
    """numpy fp64 dense masked GEMM: the page's dense-with-zeros contract."""
    md, b = c["md"], c["b"]
    W = meta.dense_weight(md["row_ptr"], md["col_idx"], c["V"].double().numpy(), c["N"], c["K"], b)
    X = c["X"].double().numpy()
    dY = c["dY"].double().numpy()
    Y = X @ W.T
    if c["bias"] is not None:
        Y = Y + c["bias"].double().numpy()[None, :]
    dX = dY @ W
    G = dY.T @ X
    mask_full = np.kron(c["mask"].astype(np.float64), np.ones((b, b)))
    Gm = G * mask_full
    # pack the masked gradient into CSR order
    dV = np.zeros((md["nnzb"], b, b))
    R = c["N"] // b
    for r in range(R):
        for i in range(md["row_ptr"][r], md["row_ptr"][r + 1]):
            cc = md["col_idx"][i]
            dV[i] = Gm[r * b:(r + 1) * b, cc * b:(cc + 1) * b]
    return Y, dX, dV, dY.sum(axis=0), Gm


def _close(a, ref, S, rel=1e-12):
    a, ref = np.asarray(a), np.asarray(ref)
    scale = np.where(S > 0, S, 1.0)
    return bool(np.all(np.abs(a - ref) <= rel * scale))


def _run_oracle(c):
    md = c["md"]
    Y, SY = oracle.fwd(c["X"], md["row_ptr"], md["col_idx"], c["V"], c["N"], c["b"], bias=c["bias"])
    dX, SX = oracle.dx(c["dY"], md["row_ptr"], md["col_idx"], c["V"], c["K"], c["b"])
    dV, SW = oracle.dw(c["dY"], c["X"], md["row_ptr"], md["col_idx"], c["b"])
    db, SB = oracle.db(c["dY"])
    return (Y, SY), (dX, SX), (dV, SW), (db, SB)


# ---------------------------------------------------------------- golden

def test_golden_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "worked_example_b2.json")))
    b, N, K = g["b"], g["N"], g["K"]
    md = meta.scan(np.array(g["mask"], dtype=np.uint8))
    V = np.array(g["V"], dtype=np.float64)
    X = np.array(g["X"], dtype=np.float64)
    dY = np.array(g["dY"], dtype=np.float64)
    Y, S = oracle.fwd(X, md["row_ptr"], md["col_idx"], V, N, b, bias=np.array(g["bias"]))
    assert np.array_equal(Y, np.array(g["Y"]))
    dX, _ = oracle.dx(dY, md["row_ptr"], md["col_idx"], V, K, b)
    assert np.array_equal(dX, np.array(g["dX"]))
    dV, _ = oracle.dw(dY, X, md["row_ptr"], md["col_idx"], b)
    assert np.array_equal(dV, np.array(g["dV"]))
    db, _ = oracle.db(dY)
    assert np.array_equal(db, np.array(g["db"]))
    assert float(np.sum((Y - np.array(g["bias"])) * dY)) == g["adjoint"]
    # S is a sum of absolute values: at least |Y - bias| + |bias|
    assert np.all(S >= np.abs(Y) - 1e-15)


def test_golden_metadata():
    g = json.load(open(os.path.join(GOLDEN, "metadata_3x4.json")))
    md = meta.scan(np.array(g["mask"], dtype=np.uint8))
    for k in ("row_ptr", "col_idx", "col_ptr", "row_idx", "perm"):
        assert md[k].tolist() == g[k], k


# ---------------------------------------------------------------- dense masked GEMM

@pytest.mark.parametrize("M,N,K,b,density,seed", [
    (128, 256, 256, 32, 0.5, 0),          # workload 1 shape
    (96, 3072, 768, 32, 0.25, 1),         # workload 2 shape, fewer rows
    (37, 192, 320, 32, 0.3, 2),           # ragged M
    (5, 256, 128, 64, 0.5, 3),            # b = 64
    (17, 24, 40, 4, 0.4, 4),              # small blocks
    (9, 12, 12, 2, 0.6, 5),
])
def test_dense_masked_gemm(M, N, K, b, density, seed):
    c = _case(M, N, K, b, density, seed)
    (Y, SY), (dX, SX), (dV, SW), (db, SB) = _run_oracle(c)
    Yd, dXd, dVd, dbd, _ = _dense_refs(c)
    assert _close(Y, Yd, SY)
    assert _close(dX, dXd, SX)
    assert _close(dV, dVd, SW)
    assert _close(db, dbd, SB)


def test_empty_rows_and_columns():
    b, R, C = 4, 5, 6
    mask = np.zeros((R, C), dtype=np.uint8)
    mask[0, 1] = mask[0, 4] = mask[3, 1] = mask[3, 2] = mask[4, 5] = 1   # rows 1, 2 and columns 0, 3 empty
    c = _case(7, R * b, C * b, b, 0, 11, mask=mask)
    (Y, SY), (dX, SX), (dV, SW), _ = _run_oracle(c)
    bias = c["bias"].double().numpy()
    for r in (1, 2):
        assert np.array_equal(Y[:, r * b:(r + 1) * b], np.broadcast_to(bias[r * b:(r + 1) * b], (7, b)))
    for cc in (0, 3):
        assert np.all(dX[:, cc * b:(cc + 1) * b] == 0)
        assert np.all(SX[:, cc * b:(cc + 1) * b] == 0)
    Yd, dXd, dVd, _, _ = _dense_refs(c)
    assert _close(Y, Yd, SY) and _close(dX, dXd, SX) and _close(dV, dVd, SW)


def test_no_blocks_at_all():
    b, R, C = 32, 3, 2
    mask = np.zeros((R, C), dtype=np.uint8)
    c = _case(4, R * b, C * b, b, 0, 12, mask=mask)
    (Y, SY), (dX, SX), (dV, _), _ = _run_oracle(c)
    assert np.array_equal(Y, np.broadcast_to(c["bias"].double().numpy(), Y.shape))
    assert np.all(dX == 0) and dV.shape == (0, b, b)


# ---------------------------------------------------------------- exact brute force

@pytest.mark.parametrize("M,N,K,b,seed", [(1, 4, 6, 2, 0), (3, 8, 4, 4, 1), (5, 6, 6, 2, 2), (3, 12, 8, 4, 3)])
def test_exact_brute_force(M, N, K, b, seed):
    """Dyadic inputs with few terms: every fp64 sum is exact, so equality is exact."""
    g = np.random.default_rng([seed, 99])
    R, C = N // b, K // b
    mask = (g.random((R, C)) < 0.6).astype(np.uint8)
    mask[0, 0] = 1
    if R > 1:
        mask[R - 1, :] = 0                      # force an empty row
    Wd = g.integers(-16, 17, size=(N, K)) / 8.0
    X = g.integers(-16, 17, size=(M, K)) / 4.0
    dY = g.integers(-16, 17, size=(M, N)) / 4.0
    bias = g.integers(-8, 9, size=(N,)) / 16.0
    md = meta.scan(mask)
    V = np.stack([Wd[r * b:(r + 1) * b, md["col_idx"][i] * b:(md["col_idx"][i] + 1) * b]
                  for r in range(R) for i in range(md["row_ptr"][r], md["row_ptr"][r + 1])]) \
        if md["nnzb"] else np.zeros((0, b, b))
    Y, _ = oracle.fwd(X, md["row_ptr"], md["col_idx"], V, N, b, bias=bias)
    assert np.array_equal(Y, np.array(brute.forward(X, Wd, mask, b, bias), dtype=np.float64))
    dX, _ = oracle.dx(dY, md["row_ptr"], md["col_idx"], V, K, b)
    assert np.array_equal(dX, np.array(brute.grad_input(dY, Wd, mask, b), dtype=np.float64))
    dV, _ = oracle.dw(dY, X, md["row_ptr"], md["col_idx"], b)
    G = np.array(brute.grad_weight_dense(dY, X, mask, b), dtype=np.float64)
    for r in range(R):
        for i in range(md["row_ptr"][r], md["row_ptr"][r + 1]):
            cc = md["col_idx"][i]
            assert np.array_equal(dV[i], G[r * b:(r + 1) * b, cc * b:(cc + 1) * b])
    # outside the kept blocks the masked dense gradient is exactly zero
    mfull = np.kron(mask, np.ones((b, b)))
    assert np.all(G[mfull == 0] == 0)
    db, _ = oracle.db(dY)
    assert np.array_equal(db, np.array(brute.grad_bias(dY), dtype=np.float64))


# ---------------------------------------------------------------- adjoint identities

@pytest.mark.parametrize("M,N,K,b,density,seed", [(64, 256, 192, 32, 0.4, 7), (11, 128, 256, 64, 0.5, 8)])
def test_adjoint_identities(M, N, K, b, density, seed):
    c = _case(M, N, K, b, density, seed, bias=True)
    (Y, SY), (dX, _), (dV, _), _ = _run_oracle(c)
    X = c["X"].double().numpy()
    dY = c["dY"].double().numpy()
    V = c["V"].double().numpy()
    lhs = np.sum((Y - c["bias"].double().numpy()[None, :]) * dY)
    mid = np.sum(X * dX)
    rhs = np.sum(dV * V)
    scale = np.sum(np.abs(SY * np.abs(dY)))
    assert abs(lhs - mid) <= 1e-12 * scale
    assert abs(lhs - rhs) <= 1e-12 * scale


# ---------------------------------------------------------------- closed forms

def test_permutation_blocks_permute_columns():
    """One identity block per block row at column sigma(r): Y[:, r-block] = X[:, sigma(r)-block] exactly."""
    b, R = 4, 6
    sigma = [3, 0, 5, 1, 4, 2]
    mask = np.zeros((R, R), dtype=np.uint8)
    for r in range(R):
        mask[r, sigma[r]] = 1
    md = meta.scan(mask)
    V = np.stack([np.eye(b)] * R)
    X = synth.activations(9, R * b, 3).double().numpy()
    Y, _ = oracle.fwd(X, md["row_ptr"], md["col_idx"], V, R * b, b)
    for r in range(R):
        assert np.array_equal(Y[:, r * b:(r + 1) * b], X[:, sigma[r] * b:(sigma[r] + 1) * b])
    # the input gradient routes back through the inverse permutation
    dY = synth.grad_output(9, R * b, 4).double().numpy()
    dX, _ = oracle.dx(dY, md["row_ptr"], md["col_idx"], V, R * b, b)
    for r in range(R):
        assert np.array_equal(dX[:, sigma[r] * b:(sigma[r] + 1) * b], dY[:, r * b:(r + 1) * b])


def test_single_block_is_plain_gemm_and_gemv():
    b = 32
    mask = np.ones((1, 1), dtype=np.uint8)
    md = meta.scan(mask)
    V = synth.block_values(1, b, 5).double().numpy()
    for M in (1, 33):
        X = synth.activations(M, b, 6).double().numpy()
        Y, S = oracle.fwd(X, md["row_ptr"], md["col_idx"], V, b, b)
        ref = X @ V[0].T if M > 1 else np.array([[float(np.dot(X[0], V[0][p])) for p in range(b)]])
        assert _close(Y, ref, S)


def test_density_one_is_dense_gemm():
    M, N, K, b = 20, 128, 96, 32
    mask = np.ones((N // b, K // b), dtype=np.uint8)
    c = _case(M, N, K, b, 1.0, 9, bias=False, mask=mask)
    (Y, SY), (dX, SX), (dV, SW), _ = _run_oracle(c)
    W = meta.dense_weight(c["md"]["row_ptr"], c["md"]["col_idx"], c["V"].double().numpy(), N, K, b)
    X, dY = c["X"].double().numpy(), c["dY"].double().numpy()
    assert _close(Y, X @ W.T, SY)
    assert _close(dX, dY @ W, SX)
    G = dY.T @ X
    assert _close(dV.reshape(N // b, K // b, b, b).transpose(0, 2, 1, 3).reshape(N, K), G,
                  SW.reshape(N // b, K // b, b, b).transpose(0, 2, 1, 3).reshape(N, K))


# ---------------------------------------------------------------- planted mistakes

def _pins_pass(fwd_fn, dx_fn, dw_fn):
    """Run the dense-masked and golden pins against possibly-mutated oracle functions."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example_b2.json")))
    md = meta.scan(np.array(g["mask"], dtype=np.uint8))
    V = np.array(g["V"], dtype=np.float64)
    X = np.array(g["X"], dtype=np.float64)
    dY = np.array(g["dY"], dtype=np.float64)
    ok = np.array_equal(fwd_fn(X, md, V, 4, 2, np.array(g["bias"])), np.array(g["Y"]))
    ok &= np.array_equal(dx_fn(dY, md, V, 4, 2), np.array(g["dX"]))
    ok &= np.array_equal(dw_fn(dY, X, md, 2), np.array(g["dV"]))
    c = _case(13, 96, 128, 32, 0.4, 21)
    Yd, dXd, dVd, _, _ = _dense_refs(c)
    m = c["md"]
    ok &= _close(fwd_fn(c["X"], m, c["V"], 96, 32, c["bias"]), Yd, np.abs(Yd) + 1)
    ok &= _close(dx_fn(c["dY"], m, c["V"], 128, 32), dXd, np.abs(dXd) + 1)
    ok &= _close(dw_fn(c["dY"], c["X"], m, 32), dVd, np.abs(dVd) + 1)
    return bool(ok)


def _good():
    f = lambda X, m, V, N, b, bias: oracle.fwd(X, m["row_ptr"], m["col_idx"], V, N, b, bias=bias)[0]
    d = lambda dY, m, V, K, b: oracle.dx(dY, m["row_ptr"], m["col_idx"], V, K, b)[0]
    w = lambda dY, X, m, b: oracle.dw(dY, X, m["row_ptr"], m["col_idx"], b)[0]
    return f, d, w


def test_pins_accept_the_oracle():
    assert _pins_pass(*_good())


def _t(V):
    V = oracle._f64(V)
    return np.ascontiguousarray(np.transpose(V, (0, 2, 1)))


@pytest.mark.parametrize("mistake", ["transposed_block", "dropped_bias", "shifted_column", "dropped_block",
                                     "dw_transposed", "dx_uses_transposed_block", "dw_wrong_operand_order"])
def test_planted_mistake_is_caught(mistake):
    f, d, w = _good()
    if mistake == "transposed_block":
        f = (lambda f0: lambda X, m, V, N, b, bias: f0(X, m, _t(V), N, b, bias))(f)
    elif mistake == "dropped_bias":
        f = (lambda f0: lambda X, m, V, N, b, bias: f0(X, m, V, N, b, None))(f)
    elif mistake == "shifted_column":
        def f(X, m, V, N, b, bias):
            ci = np.array(m["col_idx"])
            ci = np.where(ci > 0, ci - 1, ci)
            return oracle.fwd(X, m["row_ptr"], ci, V, N, b, bias=bias)[0]
    elif mistake == "dropped_block":
        def d(dY, m, V, K, b):
            V2 = oracle._f64(V).copy()
            V2[-1] = 0
            return oracle.dx(dY, m["row_ptr"], m["col_idx"], V2, K, b)[0]
    elif mistake == "dw_transposed":
        w = (lambda w0: lambda dY, X, m, b: np.ascontiguousarray(np.transpose(w0(dY, X, m, b), (0, 2, 1))))(w)
    elif mistake == "dx_uses_transposed_block":
        d = (lambda d0: lambda dY, m, V, K, b: d0(dY, m, _t(V), K, b))(d)
    elif mistake == "dw_wrong_operand_order":
        # dV computed as X^T dY restricted to the block (swapped roles of the operands)
        def w(dY, X, m, b):
            dYf, Xf = oracle._f64(dY), oracle._f64(X)
            out = []
            R = len(m["row_ptr"]) - 1
            for r in range(R):
                for i in range(m["row_ptr"][r], m["row_ptr"][r + 1]):
                    cc = m["col_idx"][i]
                    out.append(Xf[:, cc * b:(cc + 1) * b].T @ dYf[:, r * b:(r + 1) * b])
            return np.array(out)
    assert not _pins_pass(f, d, w)


# ---------------------------------------------------------------- tolerance rule

def test_tolerance_rule_flags_errors():
    ref = np.array([1.0, 0.0, -2.0])
    S = np.array([10.0, 0.0, 4.0])
    assert oracle.tolerance_check(np.array([1.03, 0.0, -2.01]), ref, S)["violations"] == 0
    assert oracle.tolerance_check(np.array([1.05, 0.0, -2.0]), ref, S)["violations"] == 1
    assert oracle.tolerance_check(np.array([1.0, 1e-30, -2.0]), ref, S)["violations"] == 1
    assert oracle.tolerance_check(np.array([np.nan, 0.0, -2.0]), ref, S)["violations"] >= 1


# ---------------------------------------------------------------- storage closed form

def test_storage_ratio_at_75_percent_sparsity():
    """Memory at 75% sparsity (pytorch_block_sparse summary, "Performance and
    Memory Efficiency": about 4x less). BSR bytes = 2 b^2 nnzb + 4 (R+1) + 4 nnzb
    for the BERT-base FFN-up workload; exact closed form 4,718,592 / 1,182,340."""
    w = synth.WORKLOADS[2]
    mask = synth.block_mask(w, 0)
    nnzb = int(mask.sum())
    assert nnzb == 576
    dense = 2 * w.N * w.K
    bsr = 2 * w.b * w.b * nnzb + 4 * (w.R + 1) + 4 * nnzb
    assert (dense, bsr) == (4718592, 1182340)
    assert 3.99 < dense / bsr < 4.0
