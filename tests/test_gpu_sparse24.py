"""GPU parity of 2:4 sparsity inside kept blocks through the C ABI against the oracle: compression
(values and index bits) and decompression are bit-exact; the forward on the sparse matrix cores
meets the layer's tolerance rule |g - ref| <= 4e-3 * S against the oracle's fp64 forward on the
oracle's decompressed blocks (exact where S = 0), and is bit-exact on integer inputs."""
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
    """N(0, 0.02) blocks with planted ties: equal magnitudes, zeros, negative zeros."""
    V = synth.block_values(nnzb, b, seed)
    if nnzb > 4:
        V[0, 0, :8] = torch.tensor([1, -1, 1, -1, 0, 0, 0, 0], dtype=torch.bfloat16)
        V[1, 2, 4:8] = torch.tensor([-0.0, 0.0, -0.0, 0.0], dtype=torch.bfloat16)
        V[2, 3, :4] = torch.tensor([0.5, 0.25, 0.5, -0.5], dtype=torch.bfloat16)
        V[3] = 0
    return V


@pytest.mark.parametrize("N,K,b,d,seed", [(256, 256, 32, 0.5, 0), (384, 640, 64, 0.4, 1), (14336, 4096, 64, 0.5, 2),
                                          (3072, 768, 32, 0.25, 3)])
def test_compress_decompress_bit_exact(N, K, b, d, seed):
    say(f"case 2:4 compress N={N} K={K} b={b} d={d}")
    mask = synth.uniform_mask(N // b, K // b, d, synth.rng(seed, synth.STREAM_PATTERN))
    p = Pattern.from_mask(mask, N, K, b)
    V = _values(p.nnzb, b, seed)
    Vc, mt = binding.values_compress_24(p, V.to(dev()))
    D = binding.values_decompress_24(p, Vc, mt)
    torch.cuda.synchronize()
    Vc_ref, mt_ref = oracle.compress_24(V)
    assert np.array_equal(mt.cpu().numpy().view(np.uint16), mt_ref)
    assert np.array_equal(Vc.cpu().view(torch.int16).numpy(),
                          torch.from_numpy(Vc_ref).to(torch.bfloat16).view(torch.int16).numpy())
    D_ref = torch.from_numpy(oracle.decompress_24(Vc_ref, mt_ref)).to(torch.bfloat16)
    assert np.array_equal(D.cpu().view(torch.int16).numpy(), D_ref.view(torch.int16).numpy())
    p.close()


@pytest.mark.parametrize("M,N,K,b,d,seed,bias", [
    (1, 256, 256, 32, 0.5, 10, True), (5, 512, 384, 64, 0.4, 11, False), (8, 1024, 512, 32, 0.3, 12, True),
    (16, 768, 512, 64, 0.5, 13, True), (17, 512, 256, 32, 0.6, 14, False), (40, 256, 512, 64, 0.5, 15, True),
    (8, 512, 512, 32, 0.02, 16, True), (3, 320, 224, 32, 0.45, 17, True)])
def test_fwd_24_matches_oracle(M, N, K, b, d, seed, bias):
    say(f"case 2:4 fwd M={M} N={N} K={K} b={b} d={d} bias={bias}")
    mask = synth.uniform_mask(N // b, K // b, d, synth.rng(seed, synth.STREAM_PATTERN))
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, N, K, b)
    V = _values(p.nnzb, b, seed)
    X = synth.activations(M, K, seed)
    bb = synth.bias_vector(N, seed) if bias else None
    Vc, mt = binding.values_compress_24(p, V.to(dev()))
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
    binding.linear_fwd_24(p, X.to(dev()), Vc, mt, None if bb is None else bb.to(dev()), out=Y)
    torch.cuda.synchronize()
    D = oracle.decompress_24(*oracle.compress_24(V))
    ref, S = oracle.fwd(X, md["row_ptr"], md["col_idx"], D, N, b, bias=bb)
    res = oracle.tolerance_check(Y.cpu(), ref, S)
    say(f"    2:4 fwd: max |g-ref|/S = {res['max_ratio']:.3e}, violations {res['violations']}")
    assert res["violations"] == 0, res
    p.close()


def test_fwd_24_decode_workload_full():
    """The decode workload at full size (X[8,4096], W[14336,4096], 64 x 64 blocks, density 0.5),
    its blocks pruned to 2:4; every output element checked."""
    w = synth.WORKLOADS[4]
    say(f"case 2:4 fwd {w.name}")
    host = synth.make_inputs(w, 0)
    md = meta.scan(host["mask"])
    p = Pattern.from_mask(host["mask"], w.N, w.K, w.b)
    Vc, mt = binding.values_compress_24(p, host["V"].to(dev()))
    Y = binding.linear_fwd_24(p, host["X"].to(dev()), Vc, mt)
    torch.cuda.synchronize()
    D = oracle.decompress_24(*oracle.compress_24(host["V"]))
    ref, S = oracle.fwd(host["X"], md["row_ptr"], md["col_idx"], D, w.N, w.b)
    res = oracle.tolerance_check(Y.cpu(), ref, S)
    say(f"    2:4 fwd: max |g-ref|/S = {res['max_ratio']:.3e}, violations {res['violations']}")
    assert res["violations"] == 0, res
    p.close()


@pytest.mark.parametrize("b", [32, 64])
def test_fwd_24_integer_inputs_bit_exact(b):
    """Integers in {-1, 0, 1}: products and fp32 sums are exact and |y| <= 256, so the output
    equals the oracle exactly."""
    M, N, K = 12, 256, 512
    g = np.random.default_rng(20 + b)
    mask = synth.uniform_mask(N // b, K // b, 0.5, g)
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, N, K, b)
    X = torch.from_numpy(g.integers(-1, 2, size=(M, K)).astype(np.float32)).to(torch.bfloat16)
    V = torch.from_numpy(g.integers(-1, 2, size=(p.nnzb, b, b)).astype(np.float32)).to(torch.bfloat16)
    Vc, mt = binding.values_compress_24(p, V.to(dev()))
    Y = binding.linear_fwd_24(p, X.to(dev()), Vc, mt)
    torch.cuda.synchronize()
    D = oracle.decompress_24(*oracle.compress_24(V))
    ref, _ = oracle.fwd(X, md["row_ptr"], md["col_idx"], D, N, b, want_s=False)
    assert np.array_equal(Y.cpu().double().numpy(), ref)
    p.close()


def test_fwd_24_argument_errors():
    mask = np.ones((2, 2), dtype=np.uint8)
    p = Pattern.from_mask(mask, 64, 64, 32)
    X = torch.zeros((4, 64), dtype=torch.bfloat16, device=dev())
    Vc = torch.zeros((4, 32, 16), dtype=torch.bfloat16, device=dev())
    mt = torch.zeros((4, 32, 2), dtype=torch.int16, device=dev())
    Y = torch.empty((4, 64), dtype=torch.bfloat16, device=dev())
    L = binding.lib()
    st = torch.cuda.current_stream().cuda_stream
    assert L.bsr_linear_fwd_24(p.handle, X.data_ptr(), 4, Vc.data_ptr(), None, None, Y.data_ptr(), st) == 1
    assert L.bsr_linear_fwd_24(p.handle, X.data_ptr(), 4, Vc.data_ptr() + 2, mt.data_ptr(), None, Y.data_ptr(),
                               st) == 3
    assert L.bsr_linear_fwd_24(p.handle, X.data_ptr(), 1 << 20, Vc.data_ptr(), mt.data_ptr(), None, Y.data_ptr(),
                               st) == 1
    p.close()


# ---- large-M forward on the sparse matrix cores (2:4 block images through the panel GEMM) ----

def _image_ref(Vc_ref: np.ndarray, mt_ref: np.ndarray, b: int) -> np.ndarray:
    """The documented image layout assembled from the oracle's compressed form (raw 16-bit units):
    per block row, the b/2 kept values, the b/16 index words, zeros to b units."""
    nnzb = Vc_ref.shape[0]
    img = np.zeros((nnzb, b, b), dtype=np.uint16)
    img[:, :, :b // 2] = torch.from_numpy(Vc_ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    img[:, :, b // 2:b // 2 + b // 16] = mt_ref
    return img


@pytest.mark.parametrize("N,K,b,d,seed", [(256, 256, 32, 0.5, 30), (384, 640, 64, 0.4, 31)])
def test_pack_24_image_layout(N, K, b, d, seed):
    mask = synth.uniform_mask(N // b, K // b, d, synth.rng(seed, synth.STREAM_PATTERN))
    p = Pattern.from_mask(mask, N, K, b)
    V = _values(p.nnzb, b, seed)
    Vc, mt = binding.values_compress_24(p, V.to(dev()))
    img = binding.values_pack_24(p, Vc, mt)
    torch.cuda.synchronize()
    Vc_ref, mt_ref = oracle.compress_24(V)
    assert np.array_equal(img.cpu().numpy().view(np.uint16), _image_ref(Vc_ref, mt_ref, b))
    p.close()


def _fwd_image(p, X, V, bias):
    Vc, mt = binding.values_compress_24(p, V)
    img = binding.values_pack_24(p, Vc, mt)
    return binding.linear_fwd_24_image(p, X, img, bias)


@pytest.mark.parametrize("variant", ["0", "1", "2", "3"])
@pytest.mark.parametrize("M,N,K,b,d,seed", [(300, 512, 480, 32, 0.4, 40), (300, 512, 448, 64, 0.4, 41),
                                            (260, 768, 256, 32, 0.8, 42), (17, 256, 512, 32, 0.5, 43),
                                            (513, 1024, 512, 32, 0.15, 44)])
def test_fwd_24_image_every_variant(monkeypatch, variant, M, N, K, b, d, seed):
    """Every panel-GEMM variant (256-row groups of 4 with 8 slots, 128-row groups of 4, 128-row
    groups of 2 and of 1) with 2:4 images, ragged row tails, half panels (K = 480), bias."""
    monkeypatch.setenv("BSR_GEMM_VARIANT", variant)
    say(f"case 2:4 image fwd variant={variant} M={M} N={N} K={K} b={b} d={d}")
    mask = synth.uniform_mask(N // b, K // b, d, synth.rng(seed, synth.STREAM_PATTERN))
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, N, K, b)
    V = _values(p.nnzb, b, seed)
    X = synth.activations(M, K, seed)
    bb = synth.bias_vector(N, seed)
    Y = _fwd_image(p, X.to(dev()), V.to(dev()), bb.to(dev()))
    torch.cuda.synchronize()
    D = oracle.decompress_24(*oracle.compress_24(V))
    ref, S = oracle.fwd(X, md["row_ptr"], md["col_idx"], D, N, b, bias=bb)
    res = oracle.tolerance_check(Y.cpu(), ref, S)
    say(f"    2:4 image fwd: max |g-ref|/S = {res['max_ratio']:.3e}, violations {res['violations']}")
    assert res["violations"] == 0, res
    p.close()


@pytest.mark.parametrize("b", [32, 64])
def test_fwd_24_image_integer_inputs_bit_exact(b):
    M, N, K = 200, 512, 512
    g = np.random.default_rng(50 + b)
    mask = synth.uniform_mask(N // b, K // b, 0.5, g)
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, N, K, b)
    X = torch.from_numpy(g.integers(-1, 2, size=(M, K)).astype(np.float32)).to(torch.bfloat16)
    V = torch.from_numpy(g.integers(-1, 2, size=(p.nnzb, b, b)).astype(np.float32)).to(torch.bfloat16)
    Y = _fwd_image(p, X.to(dev()), V.to(dev()), None)
    torch.cuda.synchronize()
    D = oracle.decompress_24(*oracle.compress_24(V))
    ref, _ = oracle.fwd(X, md["row_ptr"], md["col_idx"], D, N, b, want_s=False)
    assert np.array_equal(Y.cpu().double().numpy(), ref)
    p.close()


@pytest.mark.parametrize("k,nrows", [(2, 4096), (3, 96), (5, 64)])
def test_fwd_24_image_workloads(k, nrows):
    """The BERT-base FFN-up, square and Zipf workloads at full size with their blocks pruned to
    2:4; every row of the first, sampled rows (first, last and random) of the others."""
    w = synth.WORKLOADS[k]
    say(f"case 2:4 image fwd {w.name}")
    host = synth.make_inputs(w, 0, with_dy=False)
    md = meta.scan(host["mask"])
    p = Pattern.from_mask(host["mask"], w.N, w.K, w.b)
    Y = _fwd_image(p, host["X"].to(dev()), host["V"].to(dev()), None)
    torch.cuda.synchronize()
    g = np.random.default_rng([0, 78])
    rows = np.unique(np.concatenate([[0, w.M - 1], g.choice(w.M, size=min(nrows, w.M), replace=False)]))
    rows_t = torch.from_numpy(rows)
    D = oracle.decompress_24(*oracle.compress_24(host["V"]))
    ref, S = oracle.fwd(host["X"][rows_t], md["row_ptr"], md["col_idx"], D, w.N, w.b)
    res = oracle.tolerance_check(Y.cpu()[rows_t], ref, S)
    say(f"    2:4 image fwd ({rows.size} rows): max |g-ref|/S = {res['max_ratio']:.3e}, violations {res['violations']}")
    assert res["violations"] == 0, res
    p.close()


@pytest.mark.parametrize("b", [32, 64])
def test_24_empty_pattern_and_zero_rows(b):
    """No kept block: both 2:4 forwards give the bias exactly (NaN-poisoned outputs, small and large
    M); M = 0 enqueues nothing."""
    N, K = 4 * b, 3 * b
    mask = np.zeros((N // b, K // b), dtype=np.uint8)
    p = Pattern.from_mask(mask, N, K, b)
    V = torch.empty((0, b, b), dtype=torch.bfloat16, device=dev())
    Vc, mt = binding.values_compress_24(p, V)
    img = binding.values_pack_24(p, Vc, mt)
    bb = synth.bias_vector(N, 4).to(dev())
    for M in (5, 300):
        X = synth.activations(M, K, 4).to(dev())
        Y1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
        Y2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
        binding.linear_fwd_24(p, X, Vc, mt, bb, out=Y1)
        binding.linear_fwd_24_image(p, X, img, bb, out=Y2)
        torch.cuda.synchronize()
        assert torch.equal(Y1.cpu(), bb.cpu().expand(M, N))
        assert torch.equal(Y2.cpu(), bb.cpu().expand(M, N))
    X0 = torch.empty((0, K), dtype=torch.bfloat16, device=dev())
    binding.linear_fwd_24(p, X0, Vc, mt, bb)
    binding.linear_fwd_24_image(p, X0, img, bb)
    torch.cuda.synchronize()
    p.close()


# ---- 2:4 combined with fp8 kept values (decode forward) ----

@pytest.mark.parametrize("N,K,b,d,seed", [(256, 256, 32, 0.5, 60), (384, 640, 64, 0.4, 61), (14336, 4096, 64, 0.5, 62)])
def test_quantize_fp8_24_bit_exact(N, K, b, d, seed):
    mask = synth.uniform_mask(N // b, K // b, d, synth.rng(seed, synth.STREAM_PATTERN))
    p = Pattern.from_mask(mask, N, K, b)
    V = _values(p.nnzb, b, seed)
    Vc, mt = binding.values_compress_24(p, V.to(dev()))
    Vc8, se = binding.values_quantize_fp8_24(p, Vc)
    torch.cuda.synchronize()
    codes_ref, se_ref = oracle.quantize_fp8(oracle.compress_24(V)[0])
    assert np.array_equal(se.cpu().numpy(), se_ref)
    assert np.array_equal(Vc8.cpu().numpy(), codes_ref)
    p.close()


@pytest.mark.parametrize("M,N,K,b,d,seed,bias", [
    (1, 256, 256, 32, 0.5, 70, True), (8, 1024, 512, 32, 0.3, 71, True), (16, 768, 512, 64, 0.5, 72, False),
    (17, 512, 256, 32, 0.6, 73, False), (3, 320, 224, 32, 0.45, 74, True), (40, 256, 512, 64, 0.5, 75, True)])
def test_fwd_fp8_24_matches_oracle(M, N, K, b, d, seed, bias):
    say(f"case fp8 2:4 fwd M={M} N={N} K={K} b={b} d={d}")
    mask = synth.uniform_mask(N // b, K // b, d, synth.rng(seed, synth.STREAM_PATTERN))
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, N, K, b)
    V = _values(p.nnzb, b, seed)
    X = synth.activations(M, K, seed)
    bb = synth.bias_vector(N, seed) if bias else None
    Vc, mt = binding.values_compress_24(p, V.to(dev()))
    Vc8, se = binding.values_quantize_fp8_24(p, Vc)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
    binding.linear_fwd_fp8_24(p, X.to(dev()), Vc8, se, mt, None if bb is None else bb.to(dev()), out=Y)
    torch.cuda.synchronize()
    Vc_ref, mt_ref = oracle.compress_24(V)
    D = oracle.decompress_24(oracle.dequantize_fp8(*oracle.quantize_fp8(Vc_ref)), mt_ref)
    ref, S = oracle.fwd(X, md["row_ptr"], md["col_idx"], D, N, b, bias=bb)
    res = oracle.tolerance_check(Y.cpu(), ref, S)
    say(f"    fp8 2:4 fwd: max |g-ref|/S = {res['max_ratio']:.3e}, violations {res['violations']}")
    assert res["violations"] == 0, res
    p.close()


def test_fwd_fp8_24_decode_workload_full():
    w = synth.WORKLOADS[4]
    say(f"case fp8 2:4 fwd {w.name}")
    host = synth.make_inputs(w, 0)
    md = meta.scan(host["mask"])
    p = Pattern.from_mask(host["mask"], w.N, w.K, w.b)
    Vc, mt = binding.values_compress_24(p, host["V"].to(dev()))
    Vc8, se = binding.values_quantize_fp8_24(p, Vc)
    Y = binding.linear_fwd_fp8_24(p, host["X"].to(dev()), Vc8, se, mt)
    torch.cuda.synchronize()
    Vc_ref, mt_ref = oracle.compress_24(host["V"])
    D = oracle.decompress_24(oracle.dequantize_fp8(*oracle.quantize_fp8(Vc_ref)), mt_ref)
    ref, S = oracle.fwd(host["X"], md["row_ptr"], md["col_idx"], D, w.N, w.b)
    res = oracle.tolerance_check(Y.cpu(), ref, S)
    assert res["violations"] == 0, res
    p.close()


# ---- the wide tile on the compressed blocks (b = 32, many rows, dense groups) ----

def _mixed_mask(R, C, nfull, seed, density=0.15):
    g = np.random.default_rng(seed)
    mask = (g.random((R, C)) < density).astype(np.uint8)
    mask[g.choice(R, size=nfull, replace=False)] = 1
    mask[R - 1] = 0
    return mask


@pytest.mark.parametrize("M,R,C,nfull,seed,force", [
    (700, 20, 15, 10, 70, False),    # 3 groups (8, 8, 4 members), a last half panel, ragged row tile
    (256, 8, 16, 8, 71, False),      # one group, every sub-step dense
    (513, 33, 8, 20, 72, True),      # the last group with one member, a one-row last tile
    (300, 24, 40, 3, 73, True),      # mostly sparse rows: sub-steps with absent units
])
def test_fwd_24_wide_matches_oracle_and_image(monkeypatch, M, R, C, nfull, seed, force):
    """bsr_linear_fwd_24 through the wide tile against the oracle's forward on the decompressed
    blocks, and bit for bit against the image forward (same per-output order of sparse products)."""
    b = 32
    N, K = R * b, C * b
    mask = _mixed_mask(R, C, nfull, seed)
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, N, K, b)
    if force:
        monkeypatch.setenv("BSR_GEMM_VARIANT", "4")
    assert binding.op_kernels(p, "fwd_24", M) == ["k_wide_gemm_24"]
    say(f"case 2:4 wide fwd M={M} R={R} C={C} full={nfull} nnzb={p.nnzb}")
    V = _values(p.nnzb, b, seed)
    X = synth.activations(M, K, seed)
    bb = synth.bias_vector(N, seed)
    Vc, mt = binding.values_compress_24(p, V.to(dev()))
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
    binding.linear_fwd_24(p, X.to(dev()), Vc, mt, bb.to(dev()), out=Y)
    torch.cuda.synchronize()
    monkeypatch.delenv("BSR_GEMM_VARIANT", raising=False)
    img = binding.values_pack_24(p, Vc, mt)
    Yi = binding.linear_fwd_24_image(p, X.to(dev()), img, bb.to(dev()))
    torch.cuda.synchronize()
    assert torch.equal(Y.cpu().view(torch.int16), Yi.cpu().view(torch.int16))
    D = oracle.decompress_24(*oracle.compress_24(V))
    ref, S = oracle.fwd(X, md["row_ptr"], md["col_idx"], D, N, b, bias=bb)
    res = oracle.tolerance_check(Y.cpu(), ref, S)
    say(f"    2:4 wide fwd: max |g-ref|/S = {res['max_ratio']:.3e}, violations {res['violations']}")
    assert res["violations"] == 0, res
    p.close()


def test_fwd_24_wide_integer_inputs_bit_exact():
    """Integer activations and blocks: the wide 2:4 forward equals the oracle bit for bit."""
    M, R, C, b = 300, 16, 8, 32
    mask = _mixed_mask(R, C, 12, 74)
    g = np.random.default_rng(74)
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, R * b, C * b, b)
    assert binding.op_kernels(p, "fwd_24", M) == ["k_wide_gemm_24"]
    X = torch.from_numpy(g.integers(-2, 3, size=(M, C * b)).astype(np.float32)).to(torch.bfloat16)
    V = torch.from_numpy(g.integers(-1, 2, size=(p.nnzb, b, b)).astype(np.float32)).to(torch.bfloat16)
    Vc, mt = binding.values_compress_24(p, V.to(dev()))
    Y = binding.linear_fwd_24(p, X.to(dev()), Vc, mt)
    torch.cuda.synchronize()
    D = oracle.decompress_24(*oracle.compress_24(V))
    ref, _ = oracle.fwd(X, md["row_ptr"], md["col_idx"], D, R * b, b, want_s=False)
    assert np.array_equal(Y.cpu().double().numpy(), ref)
    p.close()


def test_fwd_24_wide_zipf_workload():
    """The Zipf 16384 x 4096 -> 11008 layer with its blocks pruned to 2:4: the wide tile takes it;
    sampled rows against the oracle, and every row bit for bit against the image forward."""
    w = synth.WORKLOADS[5]
    say(f"case 2:4 wide fwd {w.name}")
    host = synth.make_inputs(w, 0, with_dy=False)
    md = meta.scan(host["mask"])
    p = Pattern.from_mask(host["mask"], w.N, w.K, w.b)
    assert binding.op_kernels(p, "fwd_24", w.M) == ["k_wide_gemm_24"]
    Xd = host["X"].to(dev())
    Vc, mt = binding.values_compress_24(p, host["V"].to(dev()))
    Y = binding.linear_fwd_24(p, Xd, Vc, mt)
    Yi = binding.linear_fwd_24_image(p, Xd, binding.values_pack_24(p, Vc, mt))
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Yi.view(torch.int16))
    g = np.random.default_rng([0, 79])
    rows = np.unique(np.concatenate([[0, w.M - 1], g.choice(w.M, size=48, replace=False)]))
    rows_t = torch.from_numpy(rows)
    D = oracle.decompress_24(*oracle.compress_24(host["V"]))
    ref, S = oracle.fwd(host["X"][rows_t], md["row_ptr"], md["col_idx"], D, w.N, w.b)
    res = oracle.tolerance_check(Y.cpu()[rows_t], ref, S)
    say(f"    2:4 wide fwd ({rows.size} rows): max |g-ref|/S = {res['max_ratio']:.3e}, violations {res['violations']}")
    assert res["violations"] == 0, res
    p.close()


# ---- the panel GEMM staging the compressed blocks (many rows, other patterns) ----

@pytest.mark.parametrize("variant", ["0", "1", "2", "3"])
@pytest.mark.parametrize("M,N,K,b,d,seed", [(300, 512, 480, 32, 0.4, 80), (300, 512, 448, 64, 0.4, 81),
                                            (260, 768, 256, 32, 0.8, 82), (513, 1024, 512, 32, 0.15, 83),
                                            (129, 640, 384, 64, 0.3, 84)])
def test_fwd_24_compact_panel_every_variant(monkeypatch, variant, M, N, K, b, d, seed):
    """bsr_linear_fwd_24 above the few-row sizes on patterns the wide tile does not take: every
    panel-GEMM variant staging the compressed blocks, bit for bit against the image forward of the
    same variant and within the tolerance of the oracle; ragged row tails, half panels, bias."""
    monkeypatch.setenv("BSR_GEMM_VARIANT", variant)
    mask = synth.uniform_mask(N // b, K // b, d, synth.rng(seed, synth.STREAM_PATTERN))
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, N, K, b)
    assert binding.op_kernels(p, "fwd_24", M) == ["k_panel_gemm"]
    say(f"case 2:4 compact panel fwd variant={variant} M={M} N={N} K={K} b={b} d={d}")
    V = _values(p.nnzb, b, seed)
    X = synth.activations(M, K, seed).to(dev())
    bb = synth.bias_vector(N, seed).to(dev())
    Vc, mt = binding.values_compress_24(p, V.to(dev()))
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
    binding.linear_fwd_24(p, X, Vc, mt, bb, out=Y)
    Yi = binding.linear_fwd_24_image(p, X, binding.values_pack_24(p, Vc, mt), bb)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Yi.view(torch.int16))
    D = oracle.decompress_24(*oracle.compress_24(V))
    ref, S = oracle.fwd(X.cpu(), md["row_ptr"], md["col_idx"], D, N, b, bias=bb.cpu())
    res = oracle.tolerance_check(Y.cpu(), ref, S)
    say(f"    2:4 compact panel fwd: max |g-ref|/S = {res['max_ratio']:.3e}, violations {res['violations']}")
    assert res["violations"] == 0, res
    p.close()


@pytest.mark.parametrize("k", [2, 3])
def test_fwd_24_compact_panel_workloads(k):
    """The BERT-base FFN-up and square layers with their blocks pruned to 2:4 through
    bsr_linear_fwd_24: bit for bit against the image forward, sampled rows against the oracle."""
    w = synth.WORKLOADS[k]
    say(f"case 2:4 compact fwd {w.name}")
    host = synth.make_inputs(w, 0, with_dy=False)
    md = meta.scan(host["mask"])
    p = Pattern.from_mask(host["mask"], w.N, w.K, w.b)
    assert binding.op_kernels(p, "fwd_24", w.M) == ["k_panel_gemm"]
    Xd = host["X"].to(dev())
    Vc, mt = binding.values_compress_24(p, host["V"].to(dev()))
    Y = binding.linear_fwd_24(p, Xd, Vc, mt)
    Yi = binding.linear_fwd_24_image(p, Xd, binding.values_pack_24(p, Vc, mt))
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Yi.view(torch.int16))
    g = np.random.default_rng([0, 85])
    rows = np.unique(np.concatenate([[0, w.M - 1], g.choice(w.M, size=48, replace=False)]))
    rows_t = torch.from_numpy(rows)
    D = oracle.decompress_24(*oracle.compress_24(host["V"]))
    ref, S = oracle.fwd(host["X"][rows_t], md["row_ptr"], md["col_idx"], D, w.N, w.b)
    res = oracle.tolerance_check(Y.cpu()[rows_t], ref, S)
    say(f"    2:4 compact fwd ({rows.size} rows): max |g-ref|/S = {res['max_ratio']:.3e}, violations {res['violations']}")
    assert res["violations"] == 0, res
    p.close()
