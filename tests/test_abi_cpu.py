"""C-ABI checks that need no GPU: the library loads and exports every symbol the header
declares; host-only patterns give metadata bit-identical to the oracle's independent scan;
malformed input is rejected with the documented status codes. No compute call is made."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import meta
from sparse_gemm_amd import _lib, synth
from sparse_gemm_amd.binding import Pattern

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def declared_functions():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = open(os.path.join(INCLUDE, h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(bsr_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_header_declarations_are_exported():
    L = _lib.load()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.EXPORTS)
    assert L.bsr_abi_version() == 1


def test_status_strings():
    L = _lib.load()
    for code, name in _lib.STATUS.items():
        assert L.bsr_status_string(code).decode() == name
    assert L.bsr_status_string(99).decode() == "BSR_ERR_UNKNOWN"


@pytest.mark.parametrize("N,K,b,d,seed", [(256, 256, 32, 0.5, 0), (3072, 768, 32, 0.25, 1), (512, 256, 64, 0.3, 2),
                                          (64, 2048, 32, 0.05, 3), (2048, 64, 32, 1.0, 4), (128, 128, 32, 0.0, 5)])
def test_host_pattern_matches_oracle_scan(N, K, b, d, seed):
    mask = synth.uniform_mask(N // b, K // b, d, np.random.default_rng(seed))
    p = Pattern.from_mask(mask, N, K, b, upload=False)
    got = p.export()
    ref = meta.scan(mask)
    assert p.nnzb == ref["nnzb"]
    for k in ("row_ptr", "col_idx", "col_ptr", "row_idx", "perm"):
        assert np.array_equal(got[k], ref[k]), k


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_workload_patterns_match_oracle_scan(k):
    w = synth.WORKLOADS[k]
    mask = synth.block_mask(w, 0)
    p = Pattern.from_mask(mask, w.N, w.K, w.b, upload=False)
    got, ref = p.export(), meta.scan(mask)
    for key in ("row_ptr", "col_idx", "col_ptr", "row_idx", "perm"):
        assert np.array_equal(got[key], ref[key]), key


def test_csr_round_trip():
    mask = synth.uniform_mask(12, 9, 0.4, np.random.default_rng(7))
    ref = meta.scan(mask)
    p = Pattern.from_csr(12 * 32, 9 * 32, 32, ref["row_ptr"], ref["col_idx"], upload=False)
    got = p.export()
    for k in ("row_ptr", "col_idx", "col_ptr", "row_idx", "perm"):
        assert np.array_equal(got[k], ref[k]), k


def _csr_status(N, K, b, row_ptr, col_idx):
    L = _lib.load()
    rp = np.ascontiguousarray(row_ptr, dtype=np.int32)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    h = ctypes.c_void_p()
    st = L.bsr_pattern_create_from_csr(N, K, b, int(ci.size), rp.ctypes.data_as(ctypes.c_void_p),
                                       ci.ctypes.data_as(ctypes.c_void_p), 0, ctypes.byref(h))
    if st == 0:
        L.bsr_pattern_destroy(h)
    return st


@pytest.mark.parametrize("row_ptr,col_idx", [
    ([1, 2, 3], [0, 1, 0]),          # row_ptr[0] != 0
    ([0, 2, 1], [0, 1]),             # decreasing
    ([0, 2, 3], [1, 0, 0]),          # unsorted in a row
    ([0, 2, 3], [1, 1, 0]),          # duplicate in a row
    ([0, 1, 2], [0, 5]),             # column out of range
    ([0, 1, 3], [0, 1]),             # row_ptr[R] != nnzb
    ([0, 1, 2], [-1, 0]),            # negative column
])
def test_malformed_csr_rejected(row_ptr, col_idx):
    assert _csr_status(64, 128, 32, row_ptr, col_idx) == 1


def test_bad_shapes_rejected():
    L = _lib.load()
    mask = np.ones(16, dtype=np.uint8)
    h = ctypes.c_void_p()
    mk = lambda N, K, b: L.bsr_pattern_create_from_mask(N, K, b, mask.ctypes.data_as(ctypes.c_void_p), 0,
                                                        ctypes.byref(h))
    assert mk(128, 128, 16) == 2      # unsupported block size
    assert mk(100, 128, 32) == 1      # N not a multiple of b
    assert mk(0, 128, 32) == 1
    assert L.bsr_pattern_create_from_mask(64, 64, 32, None, 0, ctypes.byref(h)) == 1
    assert "mask" in L.bsr_last_error().decode()
    assert mk(128, 128, 32) == 0
    L.bsr_pattern_destroy(h)


def test_compute_on_host_only_pattern_is_refused():
    L = _lib.load()
    mask = np.ones((2, 2), dtype=np.uint8)
    p = Pattern.from_mask(mask, 64, 64, 32, upload=False)
    fake = ctypes.c_void_p(1 << 20)
    assert L.bsr_linear_fwd(p.handle, fake, 4, fake, None, fake, None) == 7
    assert L.bsr_linear_bwd_input(p.handle, fake, 4, fake, fake, None) == 7
    assert L.bsr_linear_bwd_weight(p.handle, fake, fake, 4, fake, None, None, 0, None) == 7
    assert L.bsr_linear_fwd(None, fake, 4, fake, None, fake, None) == 1


def test_workspace_query_is_host_only():
    w = synth.WORKLOADS[2]
    p = Pattern.from_mask(synth.block_mask(w, 0), w.N, w.K, w.b, upload=False)
    L = _lib.load()
    assert L.bsr_linear_bwd_weight_workspace(p.handle, 0) == 0
    assert L.bsr_linear_bwd_weight_workspace(p.handle, w.M) > 0
    assert L.bsr_linear_bwd_weight_workspace(None, w.M) == 0


# ---- host half of the block-magnitude selection: bsr_mask_topk against the oracle ----

def test_mask_topk_matches_oracle_golden():
    import json
    from oracle import convert
    from sparse_gemm_amd import binding
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "block_norms_b2.json")))
    for case in g["masks"]:
        norms = np.array(g["l1"] if case["kind"] == 1 else g["l2sq"], dtype=np.float64)
        assert np.array_equal(binding.mask_topk(norms, case["keep"]), np.array(case["mask"])), case
        assert np.array_equal(binding.mask_topk(norms, case["keep"]), convert.topk_mask(norms, case["keep"]))


@pytest.mark.parametrize("R,C,seed", [(1, 1, 0), (7, 5, 1), (96, 24, 2), (344, 128, 3)])
def test_mask_topk_matches_oracle_random(R, C, seed):
    """Bit-exact masks, with many ties (quantised norms) and with distinct norms."""
    from oracle import convert
    from sparse_gemm_amd import binding
    g = np.random.default_rng(seed)
    for quant in (True, False):
        norms = g.random((R, C))
        if quant:
            norms = np.round(norms * 8) / 8
        for keep in sorted({0, 1, (R * C) // 3, (R * C) // 2, R * C - 1, R * C}):
            if keep < 0:
                continue
            assert np.array_equal(binding.mask_topk(norms, keep), convert.topk_mask(norms, keep)), (quant, keep)


def test_mask_topk_rejects_bad_input():
    from sparse_gemm_amd import binding
    with pytest.raises(_lib.BsrError):
        binding.mask_topk(np.array([[1.0, np.nan]]), 1)
    with pytest.raises(_lib.BsrError):
        binding.mask_topk(np.ones((2, 2)), 5)
    with pytest.raises(_lib.BsrError):
        binding.mask_topk(np.ones((2, 2)), -1)
    m = binding.mask_topk(np.array([[np.inf, 1.0, np.inf]]), 1)
    assert m.tolist() == [[1, 0, 0]]


def test_pattern_size_limit():
    """A pattern holds at most 2^23 - 1 kept blocks (the weight-gradient work items pack a block's
    position into 23 bits); one more is refused with BSR_ERR_INVALID_ARG before anything is built."""
    L = _lib.load()
    b, C = 32, 128
    R = (1 << 23) // C                        # R * C = 2^23 blocks
    mask = np.ones((R, C), dtype=np.uint8)
    h = ctypes.c_void_p()
    st = L.bsr_pattern_create_from_mask(R * b, C * b, b, mask.ctypes.data_as(ctypes.c_void_p), 0, ctypes.byref(h))
    assert st == 1 and not h.value
    assert "kept blocks" in L.bsr_last_error().decode()
    mask[0, 0] = 0                            # 2^23 - 1 blocks: accepted (host only)
    p = Pattern.from_mask(mask, R * b, C * b, b, upload=False)
    assert p.nnzb == (1 << 23) - 1
    p.close()


def test_op_kernels_names_the_dispatch():
    """bsr_op_kernels (host only) names the kernels each call launches: the wide kernels for a
    pattern with full block rows at large M, the streaming small-M forward for few rows, the tile
    weight gradient (split over row chunks) for a uniform pattern; bad arguments are rejected."""
    from sparse_gemm_amd import binding
    w = synth.WORKLOADS[5]
    p = Pattern.from_mask(synth.block_mask(w, 0), w.N, w.K, w.b, upload=False)
    assert binding.op_kernels(p, "fwd", w.M) == ["k_wide_gemm"]
    assert binding.op_kernels(p, "dx", w.M) == ["k_wide_gemm"]
    assert binding.op_kernels(p, "dw", w.M) == ["k_wide_dw", "k_wide_dw_reduce"]
    assert binding.op_kernels(p, "fwd", 8) == ["k_small_m_lines"]
    assert binding.op_kernels(p, "fwd", 0) == []
    assert binding.op_kernels(p, "dw", 0) == ["k_fill_zero"]
    assert binding.op_kernels(p, "fwd_24", w.M) == ["k_wide_gemm_24"]
    assert binding.op_kernels(p, "fwd_24", 8) == ["k_fwd_24"]
    w2 = synth.WORKLOADS[2]
    p2 = Pattern.from_mask(synth.block_mask(w2, 0), w2.N, w2.K, w2.b, upload=False)
    assert binding.op_kernels(p2, "fwd", w2.M)[0] in ("k_panel_gemm", "k_wide_gemm")
    assert binding.op_kernels(p2, "dw", w2.M) == ["k_dw_panel", "k_dw_reduce"]
    assert binding.op_kernels(p2, "fwd_24", w2.M) == ["k_panel_gemm"]
    L = _lib.load()
    buf = ctypes.create_string_buffer(4)
    assert L.bsr_op_kernels(p.handle, 0, w.M, buf, 4) == 1   # too small
    assert L.bsr_op_kernels(p.handle, 4, w.M, buf, 4) == 1
    assert L.bsr_op_kernels(p.handle, 0, -1, buf, 4) == 1
    assert L.bsr_op_kernels(None, 0, 1, buf, 4) == 1


def test_weight_gradient_plan_follows_m():
    """The wide weight-gradient split is cached per pattern for the last M planned: calls with
    changing M on one pattern plan (workspace bytes, kernels) exactly as fresh patterns do."""
    from sparse_gemm_amd import binding
    w = synth.WORKLOADS[5]
    mask = synth.block_mask(w, 0)
    p = Pattern.from_mask(mask, w.N, w.K, w.b, upload=False)
    seq = [w.M, 4096, w.M, 300, 4096, 1, w.M]
    got = [(binding.bwd_weight_workspace_bytes(p, m), binding.op_kernels(p, "dw", m)) for m in seq]
    for m, g in zip(seq, got):
        q = Pattern.from_mask(mask, w.N, w.K, w.b, upload=False)
        assert g == (binding.bwd_weight_workspace_bytes(q, m), binding.op_kernels(q, "dw", m)), m
        q.close()
    # the split depends on M: 16384 rows split the sparse items over row chunks (fp32 partials and a
    # reduction), 4096 rows do not
    assert got[0][1] == ["k_wide_dw", "k_wide_dw_reduce"] and got[1][1] == ["k_wide_dw"]
    p.close()


def test_device_pattern_argument_errors():
    """bsr_pattern_create_device rejects bad shapes and capacities before touching a GPU."""
    L = _lib.load()
    h = ctypes.c_void_p()
    assert L.bsr_pattern_create_device(256, 256, 48, 10, ctypes.byref(h)) == 2    # block size
    assert L.bsr_pattern_create_device(256, 250, 32, 10, ctypes.byref(h)) == 1    # K not a multiple
    assert L.bsr_pattern_create_device(256, 256, 32, 0, ctypes.byref(h)) == 1     # cap < 1
    assert L.bsr_pattern_create_device(256, 256, 32, 65, ctypes.byref(h)) == 1    # cap > R*C
    assert L.bsr_pattern_create_device(256, 256, 32, 10, None) == 1
    assert L.bsr_pattern_rebuild(None, None, None) == 1
    host = Pattern.from_mask(np.ones((8, 8), np.uint8), 256, 256, 32, upload=False)
    ptr = ctypes.c_void_p()
    assert L.bsr_pattern_device_arrays(host.handle, ctypes.byref(ptr), None, None, None, None, None) == 2
    assert L.bsr_pattern_device_arrays(None, None, None, None, None, None, None) == 1
