"""bsr_linear_bwd_weight_noalloc (the weight gradient on the library's per-GPU scratch array, for
callers that cannot allocate): called through the C ABI, it must equal bsr_linear_bwd_weight with
a caller workspace bit for bit, and the oracle within the layer's tolerance, on two calls in a row
(the second with fewer rows, so stale scratch contents from the first are present); sizes above the
scratch array are refused."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle
from oracle import meta
from sparse_gemm_amd import _lib, binding
from sparse_gemm_amd.binding import Pattern

from gpu_util import case_inputs, check, dev, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _scratch_bytes() -> int:
    text = open(os.path.join(ROOT, "include", "bsr_linear.h")).read()
    m = re.search(r"#define BSR_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    return int(m.group(1)) << int(m.group(2))


def _noalloc(p, dY, X, dV, db):
    L = _lib.load()
    st = L.bsr_linear_bwd_weight_noalloc(p.handle, dY.data_ptr(), X.data_ptr(), dY.shape[0], dV.data_ptr(),
                                         None if db is None else db.data_ptr(),
                                         torch.cuda.current_stream().cuda_stream)
    return st


@pytest.mark.parametrize("N,K,b,d,Ms", [(3072, 768, 32, 0.25, (4096, 1000)),   # split over M (partials used)
                                        (512, 512, 64, 0.5, (700, 33)),
                                        (1024, 512, 32, 0.3, (257, 31))])
def test_noalloc_equals_workspace_call(N, K, b, d, Ms):
    host = case_inputs(max(Ms), N, K, b, 41, density=d)
    mask = host["mask"]
    md = meta.scan(mask)
    p = Pattern.from_mask(mask, N, K, b)
    for M in Ms:   # second call smaller: the scratch array still holds the first call's partials
        say(f"case noalloc dW N={N} K={K} b={b} M={M}")
        X = host["X"][:M].contiguous()
        dY = host["dY"][:M].contiguous()
        Xd, dYd = X.to(dev()), dY.to(dev())
        need = binding.bwd_weight_workspace_bytes(p, M)
        assert need <= _scratch_bytes()
        dV = torch.full((p.nnzb, b, b), float("nan"), dtype=torch.bfloat16, device=dev())
        db = torch.full((N,), float("nan"), dtype=torch.bfloat16, device=dev())
        assert _noalloc(p, dYd, Xd, dV, db) == 0, _lib.load().bsr_last_error()
        ref_dV, ref_db = binding.linear_bwd_weight(p, dYd, Xd, want_dbias=True)
        torch.cuda.synchronize()
        assert torch.equal(dV.view(torch.int16), ref_dV.view(torch.int16))
        assert torch.equal(db.view(torch.int16), ref_db.view(torch.int16))
        ref, S = oracle.dw(dY, X, md["row_ptr"], md["col_idx"], b)
        check("noalloc dV", dV, ref, S)
        ref, S = oracle.db(dY)
        check("noalloc db", db, ref, S)
    p.close()


def test_noalloc_refuses_sizes_above_the_scratch_array():
    """A pattern and M whose split-M partials need more than the scratch array: refused with
    BSR_ERR_WORKSPACE_TOO_SMALL before anything is enqueued (the outputs keep their contents)."""
    N = K = 2048
    b, M = 64, 4096   # 64 x 64 blocks at density 0.6: 5 row chunks of fp32 partials, 38.5 MiB
    host = case_inputs(M, N, K, b, 42, density=0.6)
    p = Pattern.from_mask(host["mask"], N, K, b)
    need = binding.bwd_weight_workspace_bytes(p, M)
    assert need > _scratch_bytes(), need
    Xd, dYd = host["X"].to(dev()), host["dY"].to(dev())
    dV = torch.zeros((p.nnzb, b, b), dtype=torch.bfloat16, device=dev())
    st = _noalloc(p, dYd, Xd, dV, None)
    torch.cuda.synchronize()
    assert st == 4   # BSR_ERR_WORKSPACE_TOO_SMALL
    assert "scratch" in _lib.load().bsr_last_error().decode()
    assert int(torch.count_nonzero(dV)) == 0
    p.close()
