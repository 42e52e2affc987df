"""Full-size tie-in of the three GPU ops through the adjoint identities of the layer (no bias):
<Y, dY> = <X, dX> = sum_i <dV_i, V_i>, all three equal to the sum over kept blocks of
dY[:, block row]^T X[:, block column] . V_i (the forward, input-gradient and weight-gradient
definitions, pytorch_block_sparse summary page, "Block-Sparse Implementation and Usage"; torchao
sparsity README, criteria list). Every output element of the three ops enters, not a sample.

Each inner product is taken in fp64 over the GPU's bf16 outputs. An output rounded to bf16 carries
an error of at most half a unit in its 8-bit significand, |e| <= 2^-8 |v|, and with independent
roundings of random data the error of <out, w> has standard deviation about
2^-8 / sqrt(3) * sqrt(sum (out * w)^2) (fp32 accumulation adds far less). The test allows 8 such
deviations for each side of a comparison: a statistical bound, not a worst case (on the host, with
the exact products rounded to bf16, the BERT-base gaps come to about one deviation). At the
BERT-base size one zeroed value block of dV moves its inner product by about 2 allowances and one
zeroed 32-column block of Y by about 4; at the Zipf size the allowance is wider than one block's
share, so there the identities tie the three ops together only coarsely. Element-wise parity at
these sizes is in test_gpu_parity.py."""
import math

import pytest
import torch

from sparse_gemm_amd import binding, synth
from sparse_gemm_amd.binding import Pattern

from gpu_util import dev, say

pytestmark = pytest.mark.gpu

SIGMAS = 8.0
REL = 2.0 ** -8 / math.sqrt(3.0)


def inner_and_scale(a: torch.Tensor, b: torch.Tensor, chunk: int = 1 << 24):
    """(<a, b>, sqrt(sum (a*b)^2)) in fp64 over host tensors, in chunks of elements."""
    a, b = a.reshape(-1), b.reshape(-1)
    s, q = 0.0, 0.0
    for i in range(0, a.numel(), chunk):
        prod = a[i:i + chunk].double() * b[i:i + chunk].double()
        s += float(prod.sum())
        q += float((prod * prod).sum())
    return s, math.sqrt(q)


@pytest.mark.parametrize("k", [2, 3, 5])
def test_adjoint_identities_full_size(k):
    w = synth.WORKLOADS[k]
    say(f"case adjoint identities {w.name}")
    host = synth.make_inputs(w, 0)
    p = Pattern.from_mask(host["mask"], w.N, w.K, w.b)
    X, V, dY = host["X"].to(dev()), host["V"].to(dev()), host["dY"].to(dev())
    Y = binding.linear_fwd(p, X, V)
    dX = binding.linear_bwd_input(p, dY, V)
    dV, _ = binding.linear_bwd_weight(p, dY, X)
    torch.cuda.synchronize()
    Y, dX, dV = Y.cpu(), dX.cpu(), dV.cpu()
    del X, V, dY
    a, sa = inner_and_scale(Y, host["dY"])
    b, sb = inner_and_scale(host["X"], dX)
    c, sc = inner_and_scale(dV, host["V"])
    say(f"    <Y,dY> = {a:.6e}, <X,dX> = {b:.6e}, sum <dV,V> = {c:.6e}; "
        f"rounding scales {REL * sa:.3e} / {REL * sb:.3e} / {REL * sc:.3e}")
    assert math.isfinite(a) and math.isfinite(b) and math.isfinite(c)
    assert abs(a - b) <= SIGMAS * REL * (sa + sb), (a, b)
    assert abs(b - c) <= SIGMAS * REL * (sb + sc), (b, c)
    assert abs(a - c) <= SIGMAS * REL * (sa + sc), (a, c)
    p.close()
