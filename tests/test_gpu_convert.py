"""GPU parity of the dense <-> BSR conversion and block-magnitude selection (through the C ABI)
against the oracle. All of it is integer or bit-copy work, or fp64 sums in a stated order, so
every comparison is bit-exact: block norms, the selected mask and its metadata, the gathered
block values and the dense hand-off form (raw bf16 bits)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import convert, meta
from sparse_gemm_amd import binding, synth
from sparse_gemm_amd.binding import Pattern

from gpu_util import dev, say

pytestmark = pytest.mark.gpu

# (N, K, b): small ragged grids, and the weight shapes of the reference workloads
SHAPES = [(64, 96, 32), (192, 320, 64), (3072, 768, 32), (4096, 4096, 32), (14336, 4096, 64), (11008, 4096, 32)]


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy()


@pytest.mark.parametrize("kind", [1, 2])
@pytest.mark.parametrize("N,K,b", SHAPES)
def test_block_norms_bit_exact(N, K, b, kind):
    say(f"case norms N={N} K={K} b={b} kind={kind}")
    W = synth.dense_weight(N, K, seed=N + K, b=b)
    got = binding.block_norms(W.to(dev()), b, kind)
    torch.cuda.synchronize()
    ref = oracle.block_norms(W, b, kind)
    g = got.cpu().numpy()
    assert np.array_equal(g, ref), f"{np.count_nonzero(g != ref)} norms differ"


@pytest.mark.parametrize("kind", [1, 2])
@pytest.mark.parametrize("N,K,b,d", [(64, 96, 32, 0.5), (192, 320, 64, 0.3), (3072, 768, 32, 0.25),
                                     (11008, 4096, 32, 0.3), (14336, 4096, 64, 0.5)])
def test_pattern_from_dense_matches_oracle(N, K, b, d, kind):
    say(f"case from_dense N={N} K={K} b={b} d={d} kind={kind}")
    W = synth.dense_weight(N, K, seed=7, b=b)
    R, C = N // b, K // b
    keep = int(np.floor(d * R * C + 0.5))
    p = Pattern.from_dense(W.to(dev()), b, keep, kind)
    mask = convert.topk_mask(oracle.block_norms(W, b, kind), keep)
    ref = meta.scan(mask)
    got = p.export()
    assert p.nnzb == keep == ref["nnzb"]
    for k in ("row_ptr", "col_idx", "col_ptr", "row_idx", "perm"):
        assert np.array_equal(got[k], ref[k]), k
    p.close()


def test_pattern_from_dense_ties_and_extremes():
    """A weight with many equal block norms (ties to the lower index), keep = 0 and keep = all."""
    N, K, b = 128, 256, 32
    W = torch.zeros((N, K), dtype=torch.bfloat16)
    W[:, ::3] = 0.5                     # several blocks share one norm
    W[64:96, 128:160] = -1.0
    for keep in (0, 1, 5, 17, 32):
        p = Pattern.from_dense(W.to(dev()), b, keep, 1)
        ref = meta.scan(convert.topk_mask(oracle.block_norms(W, b, 1), keep))
        got = p.export()
        assert np.array_equal(got["row_ptr"], ref["row_ptr"]) and np.array_equal(got["col_idx"], ref["col_idx"])
        p.close()


@pytest.mark.parametrize("N,K,b,d,pattern", [(64, 96, 32, 0.5, "uniform"), (320, 576, 64, 0.4, "uniform"),
                                             (3072, 768, 32, 0.25, "uniform"), (1024, 2048, 32, 0.0, "uniform"),
                                             (512, 512, 64, 1.0, "uniform"), (11008, 4096, 32, 0.3, "zipf"),
                                             (14336, 4096, 64, 0.5, "uniform")])
def test_dense_to_values_and_back_bit_exact(N, K, b, d, pattern):
    say(f"case convert N={N} K={K} b={b} d={d} {pattern}")
    g = np.random.default_rng(N * 7 + K)
    mask = (synth.zipf_mask(N // b, K // b, d, 1.1, g) if pattern == "zipf"
            else synth.uniform_mask(N // b, K // b, d, g))
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, N, K, b)
    W = synth.dense_weight(N, K, seed=3, b=b)
    Wd = W.to(dev())
    V = torch.full((p.nnzb, b, b), float("nan"), dtype=torch.bfloat16, device=dev())
    binding.dense_to_values(p, Wd, out=V)
    D = torch.full((N, K), float("nan"), dtype=torch.bfloat16, device=dev())
    binding.values_to_dense(p, V, out=D)
    torch.cuda.synchronize()
    Wb = _bits(W)
    Vref = convert.dense_to_values(Wb, md["row_ptr"], md["col_idx"], b)
    assert np.array_equal(_bits(V), Vref)
    Dref = convert.values_to_dense(Vref, md["row_ptr"], md["col_idx"], N, K, b)
    assert np.array_equal(_bits(D), Dref)
    p.close()


def test_values_to_dense_of_random_values():
    """Scatter of V that did not come from a dense weight (negative zeros kept bit for bit)."""
    N, K, b = 256, 448, 32
    mask = synth.uniform_mask(N // b, K // b, 0.4, np.random.default_rng(5))
    md = meta.scan(mask)
    V = synth.block_values(int(mask.sum()), b, 5)
    V[0, 0, :4] = -0.0
    p = Pattern.from_mask(mask, N, K, b)
    D = binding.values_to_dense(p, V.to(dev()))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(D), convert.values_to_dense(_bits(V), md["row_ptr"], md["col_idx"], N, K, b))
    p.close()


def test_layer_from_dense_by_magnitude_round_trip():
    """nn.Linear -> BlockSparseLinear by block magnitude -> to_dense equals the oracle's pruned
    weight; the layer's forward equals the dense product with it (tolerance rule)."""
    from sparse_gemm_amd.linear import BlockSparseLinear
    N, K, b, M = 512, 384, 32, 40
    lin = torch.nn.Linear(K, N, bias=True)
    W = synth.dense_weight(N, K, seed=21, b=b)
    with torch.no_grad():
        lin.weight.copy_(W.float())
        lin.bias.copy_(synth.bias_vector(N, 21).float())
    lin = lin.to(dev())
    m = BlockSparseLinear.from_dense_by_magnitude(lin, 0.3, b)
    keep = int(np.floor(0.3 * (N // b) * (K // b) + 0.5))
    mask = convert.topk_mask(oracle.block_norms(W, b, 1), keep)
    assert np.array_equal(m.block_mask(), mask)
    D = m.to_dense()
    torch.cuda.synchronize()
    kron = np.kron(mask, np.ones((b, b), dtype=np.uint8)) != 0
    assert np.array_equal(_bits(D), np.where(kron, _bits(W), 0))
    X = synth.activations(M, K, 21)
    Y = m(X.to(dev()))
    torch.cuda.synchronize()
    md = meta.scan(mask)
    Vref = convert.dense_to_values(W.double().numpy(), md["row_ptr"], md["col_idx"], b)
    ref, S = oracle.fwd(X, md["row_ptr"], md["col_idx"], Vref, N, b, bias=synth.bias_vector(N, 21))
    res = oracle.tolerance_check(Y.cpu(), ref, S)
    assert res["violations"] == 0, res


def test_convert_argument_errors():
    W = torch.zeros((64, 64), dtype=torch.bfloat16, device=dev())
    with pytest.raises(binding._lib.BsrError):
        binding.block_norms(W, 16)           # unsupported block size
    with pytest.raises(binding._lib.BsrError):
        binding.block_norms(W, 32, kind=3)
    with pytest.raises(binding._lib.BsrError):
        Pattern.from_dense(W, 32, 5)          # keep > R*C
