"""Device-built patterns (include/bsr_rebuild.h): the metadata and the compute kernels' work lists
rebuilt on the device from a device mask, so that the forward, the input gradient and the weight
gradient follow a changed mask with no host round trip (pytorch_block_sparse summary page, "Future
Development Roadmap"; pytorch/ao sparsity README, criteria list).

Each output is checked against the oracle, and bit for bit against a host-built pattern of the same
mask run in the same kernel configuration: the panel GEMM's 4-member groups (variant 1) for the
forward above 16 rows and the input gradient, the streaming forward from CSR for 16 rows or fewer,
the tile items for the weight gradient (a single row chunk below 512 rows). The value blocks past
the live count are NaN, so any read of them would show."""
import numpy as np
import pytest
import torch

import oracle
from oracle import meta
from sparse_gemm_amd import _lib, binding, synth
from sparse_gemm_amd.binding import Pattern

from gpu_util import check, dev, say

pytestmark = pytest.mark.gpu


def values_with_nan_tail(V: torch.Tensor, cap: int) -> torch.Tensor:
    out = torch.full((cap,) + tuple(V.shape[1:]), float("nan"), dtype=torch.bfloat16)
    out[: V.shape[0]] = V
    return out.to(dev())


def host_reference(mask, N, K, b, X, V, dY, M, monkeypatch):
    """Outputs of a host-built pattern of the same mask in the device pattern's configuration."""
    monkeypatch.setenv("BSR_GEMM_VARIANT", "1")
    monkeypatch.setenv("BSR_DW_TILE", "1")
    p = Pattern.from_mask(mask, N, K, b)
    Xd, Vd, dYd = X.to(dev()), V.to(dev()), dY.to(dev())
    if M <= 16:
        md = meta.scan(mask)
        rp = torch.from_numpy(md["row_ptr"]).to(dev())
        ci = torch.from_numpy(np.maximum(md["col_idx"], 0) if md["col_idx"].size else np.zeros(1, np.int32)).to(dev())
        Y = binding.linear_fwd_small_m_csr(N, K, b, rp, ci[: max(1, p.nnzb)], Xd, Vd if p.nnzb else
                                           torch.zeros((1, b, b), dtype=torch.bfloat16, device=dev()))
    else:
        Y = binding.linear_fwd(p, Xd, Vd)
    dX = binding.linear_bwd_input(p, dYd, Vd)
    dV, _ = binding.linear_bwd_weight(p, dYd, Xd)
    torch.cuda.synchronize()
    out = dict(Y=Y.cpu(), dX=dX.cpu(), dV=dV.cpu())
    p.close()
    monkeypatch.delenv("BSR_GEMM_VARIANT")
    monkeypatch.delenv("BSR_DW_TILE")
    return out


def run_device(p, mask, X, Vcap, dY):
    p.rebuild(torch.from_numpy(np.ascontiguousarray(mask.astype(np.uint8))).to(dev()))
    Y = binding.linear_fwd(p, X.to(dev()), Vcap)
    dX = binding.linear_bwd_input(p, dY.to(dev()), Vcap)
    dV, _ = binding.linear_bwd_weight(p, dY.to(dev()), X.to(dev()))
    torch.cuda.synchronize()
    return dict(Y=Y.cpu(), dX=dX.cpu(), dV=dV.cpu())


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("M,R,C,b,d,seed", [
    (300, 10, 12, 32, 0.3, 1),     # panel GEMM forward, one weight-gradient row chunk
    (8, 9, 14, 32, 0.4, 2),        # streaming forward from the device CSR
    (257, 6, 10, 64, 0.45, 3),     # 64 x 64 blocks
    (1000, 20, 9, 32, 0.15, 4),    # several weight-gradient row chunks (oracle only for dV)
    (130, 5, 40, 32, 1.0, 5),      # every block kept
])
def test_device_pattern_matches_host_pattern(monkeypatch, M, R, C, b, d, seed):
    N, K = R * b, C * b
    mask = synth.uniform_mask(R, C, d, synth.rng(seed, synth.STREAM_PATTERN))
    nnzb = int(mask.sum())
    cap = min(R * C, nnzb + 7)
    say(f"case device pattern M={M} R={R} C={C} b={b} nnzb={nnzb} cap={cap}")
    X, V, dY = synth.activations(M, K, seed), synth.block_values(nnzb, b, seed), synth.grad_output(M, N, seed)
    p = Pattern.device_built(N, K, b, cap)
    assert p.nnzb == cap
    got = run_device(p, mask, X, values_with_nan_tail(V, cap), dY)
    ref = host_reference(mask, N, K, b, X, V, dY, M, monkeypatch)
    assert same_bits(got["Y"], ref["Y"])
    assert same_bits(got["dX"], ref["dX"])
    if M < 512:
        assert same_bits(got["dV"][:nnzb], ref["dV"])
    md = meta.scan(mask)
    r, S = oracle.fwd(X, md["row_ptr"], md["col_idx"], V, N, b)
    check("fwd", got["Y"], r, S)
    r, S = oracle.dx(dY, md["row_ptr"], md["col_idx"], V, K, b)
    check("dx", got["dX"], r, S)
    r, S = oracle.dw(dY, X, md["row_ptr"], md["col_idx"], b)
    check("dw", got["dV"][:nnzb], r, S)
    assert binding.device_int(p.device_arrays()["nnzb"]) == nnzb
    p.close()


def test_device_pattern_follows_mask_changes(monkeypatch):
    """One pattern, rebuilt for masks of different densities (Zipf rows with full rows too): every
    rebuild's outputs match the host-built pattern of that mask."""
    M, R, C, b = 200, 24, 16, 32
    N, K = R * b, C * b
    g = np.random.default_rng(7)
    masks = [synth.uniform_mask(R, C, 0.5, g), synth.zipf_mask(R, C, 0.3, 1.1, g), synth.uniform_mask(R, C, 0.05, g),
             np.zeros((R, C), np.uint8), synth.uniform_mask(R, C, 0.7, g)]
    cap = max(int(m.sum()) for m in masks)
    p = Pattern.device_built(N, K, b, cap)
    X, dY = synth.activations(M, K, 7), synth.grad_output(M, N, 7)
    for k, m in enumerate(masks):
        nnzb = int(m.sum())
        say(f"  mask {k}: nnzb {nnzb}")
        V = synth.block_values(nnzb, b, 70 + k)
        got = run_device(p, m, X, values_with_nan_tail(V, cap), dY)
        if nnzb == 0:
            assert not torch.any(got["Y"].float() != 0) and not torch.any(got["dX"].float() != 0)
            continue
        ref = host_reference(m, N, K, b, X, V, dY, M, monkeypatch)
        assert same_bits(got["Y"], ref["Y"]), k
        assert same_bits(got["dX"], ref["dX"]), k
        assert same_bits(got["dV"][:nnzb], ref["dV"]), k
    p.close()


def test_device_pattern_truncates_at_capacity(monkeypatch):
    """A mask holding more blocks than the capacity: every list keeps exactly the blocks whose CSR
    position lies below cap (the forward, the input gradient and the weight gradient agree), and
    the live count reports the whole mask."""
    M, R, C, b = 160, 12, 10, 32
    N, K = R * b, C * b
    mask = synth.uniform_mask(R, C, 0.6, np.random.default_rng(9))
    nnzb = int(mask.sum())
    cap = nnzb // 2
    flat = mask.reshape(-1).copy()
    kept = np.flatnonzero(flat)
    flat[kept[cap:]] = 0          # CSR order is row-major
    trunc = flat.reshape(R, C)
    X, V, dY = synth.activations(M, K, 9), synth.block_values(cap, b, 9), synth.grad_output(M, N, 9)
    p = Pattern.device_built(N, K, b, cap)
    got = run_device(p, mask, X, V.to(dev()), dY)
    assert binding.device_int(p.device_arrays()["nnzb"]) == nnzb
    ref = host_reference(trunc, N, K, b, X, V, dY, M, monkeypatch)
    assert same_bits(got["Y"], ref["Y"])
    assert same_bits(got["dX"], ref["dX"])
    assert same_bits(got["dV"], ref["dV"])
    p.close()


def test_device_pattern_in_a_captured_graph(monkeypatch):
    """[rebuild, forward, input gradient, weight gradient] captured once and replayed for several
    masks (mask and value blocks refreshed by eager copies between replays): every replay matches
    the host-built pattern of its mask bit for bit."""
    M, R, C, b = 96, 16, 12, 32
    N, K = R * b, C * b
    g = np.random.default_rng(11)
    masks = [synth.uniform_mask(R, C, dd, g) for dd in (0.3, 0.6, 0.1)]
    cap = R * C
    X, dY = synth.activations(M, K, 11), synth.grad_output(M, N, 11)
    p = Pattern.device_built(N, K, b, cap)
    mbuf = torch.from_numpy(masks[0]).to(dev())
    vbuf = torch.zeros((cap, b, b), dtype=torch.bfloat16, device=dev())
    Xd, dYd = X.to(dev()), dY.to(dev())
    ybuf = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    dxbuf = torch.empty((M, K), dtype=torch.bfloat16, device=dev())
    dvbuf = torch.empty((cap, b, b), dtype=torch.bfloat16, device=dev())
    ws = torch.empty((max(1, binding.bwd_weight_workspace_bytes(p, M)),), dtype=torch.uint8, device=dev())

    def step():
        p.rebuild(mbuf)
        binding.linear_fwd(p, Xd, vbuf, out=ybuf)
        binding.linear_bwd_input(p, dYd, vbuf, out=dxbuf)
        binding.linear_bwd_weight(p, dYd, Xd, out=dvbuf, workspace=ws)

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for k, m in enumerate(masks + masks[:1]):
        nnzb = int(m.sum())
        V = synth.block_values(nnzb, b, 110 + k)
        mbuf.copy_(torch.from_numpy(m).to(dev()))
        vbuf.zero_()
        vbuf[:nnzb] = V.to(dev())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = host_reference(m, N, K, b, X, V, dY, M, monkeypatch)
        assert same_bits(ybuf.cpu(), ref["Y"]), k
        assert same_bits(dxbuf.cpu(), ref["dX"]), k
        assert same_bits(dvbuf[:nnzb].cpu(), ref["dV"]), k
    p.close()


def test_device_pattern_rejects_host_only_calls():
    p = Pattern.device_built(256, 256, 32, 20)
    with pytest.raises(_lib.BsrError) as e:
        p.export()
    assert e.value.status == 2
    V = torch.zeros((20, 32, 32), dtype=torch.bfloat16, device=dev())
    with pytest.raises(_lib.BsrError) as e:
        binding.values_quantize_fp8(p, V)
    assert e.value.status == 2
    h = Pattern.from_mask(np.ones((8, 8), np.uint8), 256, 256, 32)
    with pytest.raises(_lib.BsrError) as e:
        h.rebuild(torch.ones((8, 8), dtype=torch.uint8, device=dev()))
    assert e.value.status == 2
    assert binding.op_kernels(p, "fwd", 300) == ["k_panel_gemm"]
    assert binding.op_kernels(p, "fwd", 8) == ["k_small_m"]
    assert binding.op_kernels(p, "dw", 300) == ["k_dw_panel"]
    h.close()
    p.close()
