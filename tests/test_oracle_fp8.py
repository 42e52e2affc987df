"""Pins of the oracle's fp8 (OCP E4M3) block quantisation, from facts outside the oracle:
  * values of the E4M3 format fixed by the OCP 8-bit floating point specification (largest
    finite 448, smallest normal 2^-6, smallest subnormal 2^-9, the NaN codes);
  * a library routine: torch's float8_e4m3fn decoding and its round-to-nearest-even encoding;
  * brute force: the encoded code is the nearest of all finite codes, ties to the even code;
  * closed forms of the scale (the smallest power of two that brings the block into range) and
    the textbook error bound of a 3-bit mantissa;
  * the dequantised block values feed the layer's forward, which equals a dense product;
  * planted mistakes (truncation instead of rounding, a scale one power too small or too large)
    fail a pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import meta
from sparse_gemm_amd import synth

FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def test_format_constants():
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0xFE) == -448.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x38) == 1.0 and oracle.e4m3_value(0xC0) == -2.0
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    assert oracle.e4m3_value(0x00) == 0.0 and math.copysign(1.0, oracle.e4m3_value(0x80)) == -1.0


def test_decode_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        v = oracle.e4m3_value(c)
        assert (math.isnan(v) and math.isnan(ref[c])) or (v == ref[c] and math.copysign(1, v) == math.copysign(1, ref[c]))


def test_encode_matches_torch_float8_rne():
    """Random bf16 values over the whole range, every subnormal / normal midpoint, and the codes
    themselves."""
    g = np.random.default_rng(0)
    mags = np.exp2(g.uniform(-12, math.log2(448), size=4000))
    xs = list((mags * g.choice([-1, 1], size=mags.size)).astype(np.float32))
    xs = [float(torch.tensor(x).to(torch.bfloat16).double()) for x in xs]
    vals = sorted({oracle.e4m3_value(c) for c in FINITE if oracle.e4m3_value(c) >= 0})
    xs += [(a + b) / 2 for a, b in zip(vals, vals[1:])]           # every tie
    xs += [-v for v in xs[-20:]] + vals
    ref = torch.tensor(xs, dtype=torch.float64).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for x, r in zip(xs, ref):
        assert oracle.e4m3_encode(x) == int(r), (x, oracle.e4m3_encode(x), int(r))


def test_encode_is_nearest_code_brute_force():
    table = [(c, oracle.e4m3_value(c)) for c in FINITE]
    g = np.random.default_rng(1)
    for x in list(g.uniform(-448, 448, 500)) + list(g.uniform(-0.02, 0.02, 500)):
        c = oracle.e4m3_encode(x)
        best = min(abs(v - x) for _, v in table)
        assert abs(oracle.e4m3_value(c) - x) == best
        near = [cc for cc, v in table if abs(v - x) == best and math.copysign(1, v) == math.copysign(1, x)]
        if len(near) > 1:                        # a tie: the even code (last mantissa bit 0)
            assert c in near and (c & 1) == 0


def test_round_trip_of_every_code():
    for c in FINITE:
        assert oracle.e4m3_encode(oracle.e4m3_value(c)) == c


@pytest.mark.parametrize("b", [2, 32, 64])
def test_block_scale_closed_form_and_error_bound(b):
    nnzb = 40
    V = synth.block_values(nnzb, b, seed=b)
    V[3] = 0                                       # an all-zero block
    V[5] *= 1e4                                    # large magnitudes
    V[6] = V[6] * 2.0 ** -30                       # tiny magnitudes
    V[7, 0, 0] = 448.0 * 2.0 ** 5                  # amax exactly on a power-of-two boundary
    codes, se = oracle.quantize_fp8(V)
    Vd = V.double().numpy()
    deq = oracle.dequantize_fp8(codes, se)
    for i in range(nnzb):
        amax = np.abs(Vd[i]).max()
        if amax == 0:
            assert se[i] == 0 and np.all(codes[i] & 0x7F == 0)
            continue
        e = int(se[i])
        assert amax <= 448 * 2.0 ** e and (e == -126 or amax > 448 * 2.0 ** (e - 1))
        if i == 7:
            assert e == 5
        # 3-bit mantissa: relative error <= 2^-4 in the normal range, absolute <= 2^-10 below it
        a = np.abs(Vd[i])
        err = np.abs(deq[i] - Vd[i])
        normal = a >= 2.0 ** (e - 6)
        assert np.all(err[normal] <= a[normal] * 2.0 ** -4)
        assert np.all(err[~normal] <= 2.0 ** (e - 10))
        assert np.array_equal(np.signbit(deq[i][a > 0]), np.signbit(Vd[i][a > 0]))


def test_dequantized_blocks_feed_the_layer_contract():
    """Forward with the dequantised weight equals the dense product with it."""
    N, K, b, M = 256, 192, 32, 8
    mask = synth.uniform_mask(N // b, K // b, 0.5, np.random.default_rng(2))
    md = meta.scan(mask)
    V = synth.block_values(int(mask.sum()), b, 2)
    codes, se = oracle.quantize_fp8(V)
    deq = oracle.dequantize_fp8(codes, se)
    X = synth.activations(M, K, 2)
    Y, S = oracle.fwd(X, md["row_ptr"], md["col_idx"], deq, N, b)
    W = meta.dense_weight(md["row_ptr"], md["col_idx"], deq, N, K, b)
    assert np.all(np.abs(Y - X.double().numpy() @ W.T) <= 1e-12 * np.maximum(S, 1e-300))


def test_planted_mistakes_fail_a_pin():
    # truncation towards zero instead of rounding to nearest
    x = 1.1875                                     # between 1.125 and 1.25, nearer 1.25
    trunc = 0x38 | int(((x - 1.0) * 8))            # 1.125
    assert oracle.e4m3_encode(x) != trunc
    # the scale pin accepts only the smallest power of two: e = 0 for amax = 300
    amax = 300.0
    _, se = oracle.quantize_fp8(torch.full((1, 2, 2), amax).to(torch.bfloat16))
    assert int(se[0]) == 0

    def scale_pin(e):
        return amax <= 448 * 2.0 ** e and amax > 448 * 2.0 ** (e - 1)
    assert scale_pin(0) and not scale_pin(-1) and not scale_pin(1)


def test_fp8_of_24_kept_values():
    """fp8 codes of the kept values of 2:4 blocks: every group keeps its largest magnitude, so a
    block's scale exponent is the same whether taken over the block or over its kept values; the
    forward with the dequantised, decompressed blocks equals the dense product with them."""
    N, K, b, M = 256, 256, 32, 6
    mask = synth.uniform_mask(N // b, K // b, 0.5, np.random.default_rng(5))
    md = meta.scan(mask)
    V = synth.block_values(int(mask.sum()), b, 5)
    V[0] *= 1e3
    V[1] = V[1] * 2.0 ** -20
    Vc, mt = oracle.compress_24(V)
    codes, se = oracle.quantize_fp8(Vc)
    assert codes.shape == Vc.shape
    assert np.array_equal(se, oracle.quantize_fp8(V)[1])
    D = oracle.decompress_24(oracle.dequantize_fp8(codes, se), mt)
    X = synth.activations(M, K, 5)
    Y, S = oracle.fwd(X, md["row_ptr"], md["col_idx"], D, N, b)
    W = meta.dense_weight(md["row_ptr"], md["col_idx"], D, N, K, b)
    assert np.all(np.abs(Y - X.double().numpy() @ W.T) <= 1e-12 * np.maximum(S, 1e-300))
