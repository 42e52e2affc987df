"""BlockSparseLinear as a drop-in nn.Linear trained as usual (pytorch_block_sparse summary page,
"Block-Sparse Implementation and Usage"; the pattern stays fixed, "Future Development Roadmap"):
gradients from loss.backward() against the fp64 oracle, a few SGD steps that keep the pattern, and
a state_dict round trip into a fresh module that reproduces the outputs bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from oracle import meta
from sparse_gemm_amd import synth
from sparse_gemm_amd.linear import BlockSparseLinear

from gpu_util import check, dev, say

pytestmark = pytest.mark.gpu


def _layer(K, N, b, density, seed, bias=True):
    m = BlockSparseLinear(K, N, bias=bias, density=density, block_size=b, seed=seed, device=dev())
    with torch.no_grad():
        m.values.copy_(synth.block_values(m.pattern.nnzb, b, seed).to(dev()))
        if bias:
            m.bias.copy_(synth.bias_vector(N, seed).to(dev()))
    return m


@pytest.mark.parametrize("M,K,N,b,density", [(96, 256, 384, 32, 0.4), (300, 512, 256, 64, 0.5),
                                              (20, 768, 3072, 32, 0.25)])
def test_backward_matches_oracle(M, K, N, b, density):
    """x.grad, values.grad and bias.grad from loss.backward() with loss = <y, dY> (so dL/dy = dY)
    equal the oracle's dX, dV and db within the layer's tolerance."""
    say(f"case layer backward M={M} K={K} N={N} b={b} d={density}")
    seed = 31
    m = _layer(K, N, b, density, seed)
    X = synth.activations(M, K, seed)
    dY = synth.grad_output(M, N, seed)
    x = X.to(dev()).requires_grad_(True)
    y = m(x)
    loss = (y.float() * dY.to(dev()).float()).sum()
    loss.backward()
    torch.cuda.synchronize()
    mask = m.block_mask()
    md = meta.scan(mask)
    V = m.values.detach().cpu()
    ref, S = oracle.fwd(X, md["row_ptr"], md["col_idx"], V, N, b, bias=m.bias.detach().cpu())
    check("layer fwd", y.detach(), ref, S)
    ref, S = oracle.dx(dY, md["row_ptr"], md["col_idx"], V, K, b)
    check("x.grad", x.grad, ref, S)
    ref, S = oracle.dw(dY, X, md["row_ptr"], md["col_idx"], b)
    check("values.grad", m.values.grad, ref, S)
    ref, S = oracle.db(dY)
    check("bias.grad", m.bias.grad, ref, S)


def test_batched_input_and_no_bias():
    """A 3-D input [batch, seq, K] is flattened to rows and restored; without a bias only x and the
    values get gradients."""
    b, K, N = 32, 256, 256
    m = _layer(K, N, b, 0.5, 32, bias=False)
    X = synth.activations(2 * 24, K, 32)
    x = X.reshape(2, 24, K).to(dev()).requires_grad_(True)
    y = m(x)
    assert y.shape == (2, 24, N)
    dY = synth.grad_output(48, N, 32)
    y.backward(dY.reshape(2, 24, N).to(dev()))
    torch.cuda.synchronize()
    md = meta.scan(m.block_mask())
    V = m.values.detach().cpu()
    ref, S = oracle.dx(dY, md["row_ptr"], md["col_idx"], V, K, b)
    check("x.grad (3-D)", x.grad.reshape(48, K), ref, S)
    ref, S = oracle.dw(dY, X, md["row_ptr"], md["col_idx"], b)
    check("values.grad (3-D)", m.values.grad, ref, S)


def test_sgd_steps_keep_the_pattern():
    """Three SGD steps change the block values, never the pattern; after them the forward still
    equals the oracle on the updated values."""
    M, K, N, b = 64, 256, 512, 32
    m = _layer(K, N, b, 0.3, 33)
    meta0 = m.pattern.export()
    rp0, ci0 = m.row_ptr.clone(), m.col_idx.clone()
    opt = torch.optim.SGD(m.parameters(), lr=0.05)
    X = synth.activations(M, K, 33).to(dev())
    v0 = m.values.detach().clone()
    for step in range(3):
        opt.zero_grad()
        y = m(X)
        loss = (y.float() ** 2).mean()
        loss.backward()
        opt.step()
    torch.cuda.synchronize()
    meta1 = m.pattern.export()
    for k in meta0:
        assert np.array_equal(meta0[k], meta1[k]), k
    assert torch.equal(m.row_ptr, rp0) and torch.equal(m.col_idx, ci0)
    assert m.values.shape == v0.shape and not torch.equal(m.values.detach(), v0)
    md = meta.scan(m.block_mask())
    y = m(X).detach()
    torch.cuda.synchronize()
    ref, S = oracle.fwd(X.cpu(), md["row_ptr"], md["col_idx"], m.values.detach().cpu(), N, b,
                        bias=m.bias.detach().cpu())
    check("fwd after SGD", y, ref, S)


def test_state_dict_round_trip_is_bit_exact():
    """state_dict -> a fresh module built with another pattern -> load_state_dict: the fresh module
    takes the saved pattern and values, and its outputs and gradients equal the original's bit for
    bit. Its `values` stays the same Parameter object (an optimizer built before the load keeps
    updating it)."""
    M, K, N, b = 80, 384, 256, 32
    a = _layer(K, N, b, 0.35, 34)
    X = synth.activations(M, K, 34).to(dev())
    sd = {k: v.detach().clone() for k, v in a.state_dict().items()}
    fresh = BlockSparseLinear(K, N, bias=True, density=0.7, block_size=b, seed=99, device=dev())
    param = fresh.values
    opt = torch.optim.SGD(fresh.parameters(), lr=0.1)
    fresh.load_state_dict(sd)
    assert fresh.values is param
    assert fresh.values.shape == a.values.shape
    assert np.array_equal(fresh.block_mask(), a.block_mask())
    xa, xf = X.clone().requires_grad_(True), X.clone().requires_grad_(True)
    ya, yf = a(xa), fresh(xf)
    dY = synth.grad_output(M, N, 34).to(dev())
    ya.backward(dY)
    yf.backward(dY)
    torch.cuda.synchronize()
    assert torch.equal(ya, yf)
    assert torch.equal(xa.grad, xf.grad)
    assert torch.equal(a.values.grad, fresh.values.grad)
    assert torch.equal(a.bias.grad, fresh.bias.grad)
    before = fresh.values.detach().clone()
    opt.step()
    assert not torch.equal(fresh.values.detach(), before)   # the earlier optimizer reaches the new values
