"""GPU parity of the fp8 (OCP E4M3) block values through the C ABI against the oracle:
quantisation (codes and scale exponents) and dequantisation are bit-exact; the fp8 forward
meets the layer's tolerance rule |g - ref| <= 4e-3 * S against the oracle's fp64 forward on the
oracle's dequantised weight (exact where S = 0: rows with no kept block give the bias)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import meta
from sparse_gemm_amd import binding, synth
from sparse_gemm_amd.binding import Pattern

from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _values(nnzb, b, seed):
    """N(0, 0.02) blocks, some with other magnitudes, one all zero, negative zeros."""
    V = synth.block_values(nnzb, b, seed)
    if nnzb > 8:
        V[1] = V[1] * 3e3
        V[2] = V[2] * 2.0 ** -40
        V[3] = 0
        V[4, 0, :3] = -0.0
        V[5, 1, 1] = 448.0          # amax on a power-of-two boundary of the scale
    return V


@pytest.mark.parametrize("N,K,b,d,seed", [(256, 256, 32, 0.5, 0), (384, 640, 64, 0.4, 1), (14336, 4096, 64, 0.5, 2),
                                          (3072, 768, 32, 0.25, 3)])
def test_quantize_and_dequantize_bit_exact(N, K, b, d, seed):
    say(f"case fp8 quantize N={N} K={K} b={b} d={d}")
    mask = synth.uniform_mask(N // b, K // b, d, synth.rng(seed, synth.STREAM_PATTERN))
    p = Pattern.from_mask(mask, N, K, b)
    V = _values(p.nnzb, b, seed)
    V8, se = binding.values_quantize_fp8(p, V.to(dev()))
    Vd = binding.values_dequantize_fp8(p, V8, se)
    torch.cuda.synchronize()
    codes_ref, se_ref = oracle.quantize_fp8(V)
    assert np.array_equal(se.cpu().numpy(), se_ref)
    assert np.array_equal(V8.cpu().numpy(), codes_ref), f"{np.count_nonzero(V8.cpu().numpy() != codes_ref)} codes"
    deq = oracle.dequantize_fp8(codes_ref, se_ref)
    ref_bits = torch.from_numpy(deq).to(torch.bfloat16)
    assert torch.equal(ref_bits.double(), torch.from_numpy(deq)), "dequantised values not bf16 values"
    assert np.array_equal(Vd.cpu().view(torch.int16).numpy(), ref_bits.view(torch.int16).numpy())
    p.close()


@pytest.mark.parametrize("M,N,K,b,d,seed,bias", [
    (1, 256, 256, 32, 0.5, 10, True), (5, 512, 384, 64, 0.4, 11, False), (8, 1024, 512, 32, 0.3, 12, True),
    (16, 768, 512, 64, 0.5, 13, True), (17, 512, 256, 32, 0.6, 14, False), (40, 256, 512, 64, 0.5, 15, True),
    (8, 512, 512, 32, 0.02, 16, True)])
def test_fwd_fp8_matches_oracle(M, N, K, b, d, seed, bias):
    say(f"case fp8 fwd M={M} N={N} K={K} b={b} d={d} bias={bias}")
    mask = synth.uniform_mask(N // b, K // b, d, synth.rng(seed, synth.STREAM_PATTERN))
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, N, K, b)
    V = _values(p.nnzb, b, seed)
    X = synth.activations(M, K, seed)
    bb = synth.bias_vector(N, seed) if bias else None
    V8, se = binding.values_quantize_fp8(p, V.to(dev()))
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
    binding.linear_fwd_fp8(p, X.to(dev()), V8, se, None if bb is None else bb.to(dev()), out=Y)
    torch.cuda.synchronize()
    deq = oracle.dequantize_fp8(*oracle.quantize_fp8(V))
    ref, S = oracle.fwd(X, md["row_ptr"], md["col_idx"], deq, N, b, bias=bb)
    res = oracle.tolerance_check(Y.cpu(), ref, S)
    say(f"    fp8 fwd: max |g-ref|/S = {res['max_ratio']:.3e}, violations {res['violations']}")
    assert res["violations"] == 0, res
    p.close()


def test_fwd_fp8_decode_workload_full():
    """The decode workload at full size: X[8,4096], W[14336,4096], 64 x 64 blocks, density 0.5,
    every output element checked."""
    w = synth.WORKLOADS[4]
    say(f"case fp8 fwd {w.name}")
    host = synth.make_inputs(w, 0)
    md = meta.scan(host["mask"])
    p = Pattern.from_mask(host["mask"], w.N, w.K, w.b)
    V8, se = binding.values_quantize_fp8(p, host["V"].to(dev()))
    Y = binding.linear_fwd_fp8(p, host["X"].to(dev()), V8, se)
    torch.cuda.synchronize()
    deq = oracle.dequantize_fp8(*oracle.quantize_fp8(host["V"]))
    ref, S = oracle.fwd(host["X"], md["row_ptr"], md["col_idx"], deq, w.N, w.b)
    res = oracle.tolerance_check(Y.cpu(), ref, S)
    say(f"    fp8 fwd: max |g-ref|/S = {res['max_ratio']:.3e}, violations {res['violations']}")
    assert res["violations"] == 0, res
    # the fp8 layer stays close to the bf16 layer: each weight moves by at most 2^-4 of itself in
    # the normal range (a little more relative to the rounded value), so |Y8 - Y16| <= 2^-3 S
    ref16, _ = oracle.fwd(host["X"], md["row_ptr"], md["col_idx"], host["V"], w.N, w.b, want_s=False)
    assert np.all(np.abs(ref - ref16) <= 2.0 ** -3 * S)
    p.close()


def test_fwd_fp8_integer_inputs_bit_exact():
    """Small integers in X and in the block values: every product and partial sum is exact in
    fp32 and the results are integers below 256, so the output must equal the oracle exactly."""
    M, N, K, b = 12, 256, 256, 32
    g = np.random.default_rng(20)
    mask = synth.uniform_mask(N // b, K // b, 0.5, g)
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, N, K, b)
    X = torch.from_numpy(g.integers(-1, 2, size=(M, K)).astype(np.float32)).to(torch.bfloat16)
    V = torch.from_numpy(g.integers(-1, 2, size=(p.nnzb, b, b)).astype(np.float32)).to(torch.bfloat16)
    V8, se = binding.values_quantize_fp8(p, V.to(dev()))
    Y = binding.linear_fwd_fp8(p, X.to(dev()), V8, se)
    torch.cuda.synchronize()
    ref, _ = oracle.fwd(X, md["row_ptr"], md["col_idx"], V, N, b, want_s=False)
    assert np.array_equal(Y.cpu().double().numpy(), ref)
    p.close()


def test_fwd_fp8_argument_errors():
    mask = np.ones((2, 2), dtype=np.uint8)
    p = Pattern.from_mask(mask, 64, 64, 32)
    X = torch.zeros((4, 64), dtype=torch.bfloat16, device=dev())
    V8 = torch.zeros((4, 32, 32), dtype=torch.uint8, device=dev())
    se = torch.zeros((4,), dtype=torch.int32, device=dev())
    Y = torch.empty((4, 64), dtype=torch.bfloat16, device=dev())
    L = binding.lib()
    st = torch.cuda.current_stream().cuda_stream
    assert L.bsr_linear_fwd_fp8(p.handle, X.data_ptr(), 4, V8.data_ptr(), None, None, Y.data_ptr(), st) != 0
    assert L.bsr_linear_fwd_fp8(p.handle, X.data_ptr(), 4, V8.data_ptr(), se.data_ptr() + 2, None, Y.data_ptr(),
                                st) == 3
    assert L.bsr_linear_fwd_fp8(p.handle, X.data_ptr(), 1 << 20, V8.data_ptr(), se.data_ptr(), None, Y.data_ptr(),
                                st) == 1
    assert L.bsr_linear_fwd_fp8(p.handle, X.data_ptr(), 0, V8.data_ptr(), se.data_ptr(), None, Y.data_ptr(), st) == 0
    p.close()


@pytest.mark.parametrize("b", [32, 64])
def test_fp8_empty_pattern_and_zero_rows(b):
    """No kept block: quantisation does nothing and the forward gives the bias exactly (NaN-poisoned
    output); M = 0 enqueues nothing."""
    N, K, M = 4 * b, 3 * b, 5
    mask = np.zeros((N // b, K // b), dtype=np.uint8)
    p = Pattern.from_mask(mask, N, K, b)
    V = torch.empty((0, b, b), dtype=torch.bfloat16, device=dev())
    V8, se = binding.values_quantize_fp8(p, V)
    bb = synth.bias_vector(N, 3).to(dev())
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
    binding.linear_fwd_fp8(p, synth.activations(M, K, 3).to(dev()), V8, se, bb, out=Y)
    binding.linear_fwd_fp8(p, torch.empty((0, K), dtype=torch.bfloat16, device=dev()), V8, se, bb)
    torch.cuda.synchronize()
    assert torch.equal(Y.cpu(), bb.cpu().expand(M, N))
    p.close()
