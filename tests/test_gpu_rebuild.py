"""GPU parity of the on-device metadata rebuild (bsr_meta_rebuild) against the oracle's scan of
the mask: row_ptr, col_idx, col_ptr, row_idx, perm and nnzb bit-exact, for uniform and Zipf masks,
empty rows and columns, all-zero and full masks, grids wider and taller than one work-group's
pass, a capacity below nnzb, and replays of a captured HIP graph with the mask changed between
them."""
import numpy as np
import pytest
import torch

from oracle import meta
from sparse_gemm_amd import binding, synth

from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _check(mask: np.ndarray, out: dict) -> None:
    ref = meta.scan(mask)
    n = ref["nnzb"]
    assert int(out["nnzb"].item()) == n
    assert np.array_equal(out["row_ptr"].cpu().numpy(), ref["row_ptr"])
    assert np.array_equal(out["col_ptr"].cpu().numpy(), ref["col_ptr"])
    for k in ("col_idx", "row_idx", "perm"):
        assert np.array_equal(out[k].cpu().numpy()[:n], ref[k]), k


def _masks():
    g = np.random.default_rng(0)
    yield "uniform 96x24 d0.25", synth.uniform_mask(96, 24, 0.25, g)
    yield "uniform 128x128 d0.10", synth.uniform_mask(128, 128, 0.10, g)
    yield "zipf 344x128 d0.30", synth.zipf_mask(344, 128, 0.30, 1.1, g)
    yield "uniform 224x64 d0.5", synth.uniform_mask(224, 64, 0.5, g)
    yield "wide 3x700 d0.3", synth.uniform_mask(3, 700, 0.3, g)
    yield "tall 600x5 d0.4", synth.uniform_mask(600, 5, 0.4, g)
    m = synth.uniform_mask(40, 30, 0.4, g)
    m[7] = 0
    m[:, 11] = 0
    yield "empty row and column", m
    yield "all zero", np.zeros((17, 9), dtype=np.uint8)
    yield "full", np.ones((33, 65), dtype=np.uint8)
    yield "1x1 kept", np.ones((1, 1), dtype=np.uint8)
    yield "1x1 empty", np.zeros((1, 1), dtype=np.uint8)


@pytest.mark.parametrize("name,mask", list(_masks()), ids=[n for n, _ in _masks()])
def test_rebuild_bit_exact(name, mask):
    say(f"case rebuild {name}")
    out = binding.meta_rebuild(torch.from_numpy(mask).to(dev()))
    torch.cuda.synchronize()
    _check(mask, out)


def test_rebuild_capacity_below_nnzb():
    mask = synth.uniform_mask(20, 20, 0.5, np.random.default_rng(1))
    n = int(mask.sum())
    cap = n // 3
    out = binding.meta_rebuild(torch.from_numpy(mask).to(dev()), cap=cap)
    torch.cuda.synchronize()
    ref = meta.scan(mask)
    assert int(out["nnzb"].item()) == n
    assert np.array_equal(out["row_ptr"].cpu().numpy(), ref["row_ptr"])
    assert np.array_equal(out["col_idx"].cpu().numpy()[:cap], ref["col_idx"][:cap])
    # CSC entries below cap are exact, the rest are not written (arrays have length cap)
    assert np.array_equal(out["row_idx"].cpu().numpy()[:cap], ref["row_idx"][:cap])
    assert np.array_equal(out["perm"].cpu().numpy()[:cap], ref["perm"][:cap])


def test_rebuild_feeds_a_pattern():
    """CSR rebuilt on the device, copied to the host, gives a pattern equal to the one built from
    the mask (and usable by the compute calls)."""
    w = synth.WORKLOADS[2]
    mask = synth.block_mask(w, 3)
    out = binding.meta_rebuild(torch.from_numpy(mask).to(dev()))
    torch.cuda.synchronize()
    n = int(out["nnzb"].item())
    p = binding.Pattern.from_csr(w.N, w.K, w.b, out["row_ptr"].cpu().numpy(), out["col_idx"].cpu().numpy()[:n])
    q = binding.Pattern.from_mask(mask, w.N, w.K, w.b)
    a, b = p.export(), q.export()
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    p.close()
    q.close()


def test_rebuild_in_a_captured_graph_with_changing_masks():
    R, C = 96, 48
    g = np.random.default_rng(2)
    masks = [synth.uniform_mask(R, C, d, g) for d in (0.2, 0.5, 0.05, 0.9)]
    buf = torch.from_numpy(masks[0]).to(dev())
    out = binding.meta_rebuild(buf)          # eager run: also allocates the outputs
    torch.cuda.synchronize()
    _check(masks[0], out)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        binding.meta_rebuild(buf)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        gout = binding.meta_rebuild(buf)
    for m in masks[1:] + masks[:1]:
        buf.copy_(torch.from_numpy(m).to(dev()))   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _check(m, gout)
        eager = binding.meta_rebuild(buf)
        torch.cuda.synchronize()
        _check(m, eager)


def test_rebuild_argument_errors():
    L = binding.lib()
    mask = torch.zeros((4, 4), dtype=torch.uint8, device=dev())
    i32 = torch.zeros(64, dtype=torch.int32, device=dev())
    ws = torch.zeros(int(L.bsr_meta_rebuild_workspace(4, 4)), dtype=torch.uint8, device=dev())
    st = torch.cuda.current_stream().cuda_stream
    p = i32.data_ptr()
    assert L.bsr_meta_rebuild(0, 4, mask.data_ptr(), p, p, p, p, p, 16, p, ws.data_ptr(), ws.numel(), st) == 1
    assert L.bsr_meta_rebuild(4, 4, mask.data_ptr(), p, p, p, p, p, 16, p, ws.data_ptr(), 8, st) == 4
    assert L.bsr_meta_rebuild(4, 4, mask.data_ptr(), p + 2, p, p, p, p, 16, p, ws.data_ptr(), ws.numel(), st) == 3
    assert L.bsr_meta_rebuild(4, 4, None, p, p, p, p, p, 16, p, ws.data_ptr(), ws.numel(), st) == 1


# ---- the small-M forward straight from device-rebuilt metadata ----

@pytest.mark.parametrize("M,N,K,b,d,seed", [(8, 512, 512, 64, 0.5, 100), (1, 256, 384, 32, 0.3, 101),
                                            (16, 3072, 768, 32, 0.25, 102), (5, 384, 256, 64, 0.0, 103)])
def test_fwd_small_m_from_rebuilt_csr(monkeypatch, M, N, K, b, d, seed):
    """Mask -> bsr_meta_rebuild -> bsr_linear_fwd_small_m_csr, all on the device: equals the oracle
    (tolerance rule) and, bit for bit, the host-scheduled forward in the configuration with the same
    blocks per wave (for b = 32 the streaming kernel's 8 blocks per wave and pass, configuration 3;
    for b = 64 the default's one block per wave and pass)."""
    if b == 32:
        monkeypatch.setenv("BSR_SMALLM_CONFIG", "3")
    say(f"case small-M from device CSR M={M} N={N} K={K} b={b} d={d}")
    from gpu_util import case_inputs
    host = case_inputs(M, N, K, b, seed, density=d, bias=True, dy=False)
    mask = host["mask"]
    md = meta.scan(mask)
    out = binding.meta_rebuild(torch.from_numpy(mask).to(dev()))
    X, V, bias = host["X"].to(dev()), host["V"].to(dev()), host["bias"].to(dev())
    Vpad = torch.zeros((max(1, V.shape[0]), b, b), dtype=torch.bfloat16, device=dev())
    Vpad[:V.shape[0]] = V
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
    binding.linear_fwd_small_m_csr(N, K, b, out["row_ptr"], out["col_idx"], X, Vpad, bias, out=Y)
    p = binding.Pattern.from_mask(mask, N, K, b)
    Yh = binding.linear_fwd(p, X, V, bias)
    torch.cuda.synchronize()
    import oracle
    ref, S = oracle.fwd(host["X"], md["row_ptr"], md["col_idx"], host["V"], N, b, bias=host["bias"])
    res = oracle.tolerance_check(Y.cpu(), ref, S)
    assert res["violations"] == 0, res
    assert torch.equal(Y.cpu(), Yh.cpu())
    p.close()


@pytest.mark.parametrize("M,N,K,b,seed", [(8, 512, 512, 64, 110), (16, 1024, 768, 32, 111), (3, 384, 256, 32, 112)])
def test_fwd_small_m_from_csr_truncated_at_capacity(M, N, K, b, seed):
    """A mask rebuilt past its capacity: row_ptr is written in full but col_idx only below cap, and V
    holds cap blocks. The forward keeps each row's blocks below cap and drops the rest (never reading
    past col_idx or V): it must equal the oracle on the CSR truncated at cap."""
    say(f"case small-M from device CSR truncated at cap M={M} N={N} K={K} b={b}")
    import oracle
    from gpu_util import case_inputs
    host = case_inputs(M, N, K, b, seed, density=0.6, bias=True, dy=False)
    mask = host["mask"]
    md = meta.scan(mask)
    n = md["nnzb"]
    cap = n // 2 + 1
    out = binding.meta_rebuild(torch.from_numpy(mask).to(dev()), cap=cap)
    assert int(out["nnzb"].item()) == n > cap
    X, bias = host["X"].to(dev()), host["bias"].to(dev())
    Vcap = host["V"][:cap].contiguous()
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
    binding.linear_fwd_small_m_csr(N, K, b, out["row_ptr"], out["col_idx"], X, Vcap.to(dev()), bias, out=Y)
    torch.cuda.synchronize()
    rp = np.minimum(md["row_ptr"], cap).astype(np.int32)
    ref, S = oracle.fwd(host["X"], rp, md["col_idx"][:cap], Vcap, N, b, bias=host["bias"])
    res = oracle.tolerance_check(Y.cpu(), ref, S)
    assert res["violations"] == 0, res


def test_changing_mask_to_forward_in_one_captured_graph():
    """A captured graph of [rebuild the metadata of the current mask, forward from it] replayed for
    several masks (mask and block values refreshed by eager copies between replays): every replay
    matches the oracle."""
    import oracle
    M, N, K, b = 8, 512, 256, 32
    R, C = N // b, K // b
    g = np.random.default_rng(104)
    masks = [synth.uniform_mask(R, C, dd, g) for dd in (0.3, 0.6, 0.1)]
    X = synth.activations(M, K, 104)
    mbuf = torch.from_numpy(masks[0]).to(dev())
    vbuf = torch.zeros((R * C, b, b), dtype=torch.bfloat16, device=dev())
    Xd = X.to(dev())
    ybuf = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    def step():
        o = binding.meta_rebuild(mbuf)
        binding.linear_fwd_small_m_csr(N, K, b, o["row_ptr"], o["col_idx"], Xd, vbuf, None, out=ybuf)
        return o
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
        V = synth.block_values(int(m.sum()), b, 200 + k)
        mbuf.copy_(torch.from_numpy(m).to(dev()))
        vbuf.zero_()
        vbuf[:V.shape[0]] = V.to(dev())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        md = meta.scan(m)
        ref, S = oracle.fwd(X, md["row_ptr"], md["col_idx"], V, N, b)
        res = oracle.tolerance_check(ybuf.cpu(), ref, S)
        assert res["violations"] == 0, (k, res)
