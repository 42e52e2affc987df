"""Helpers for the GPU parity tests: seeded inputs on the device, oracle comparisons."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from oracle import meta
from sparse_gemm_amd import binding, synth
from sparse_gemm_amd.binding import Pattern


def say(*a) -> None:
    print(*a, flush=True)
    sys.stdout.flush()


def dev() -> torch.device:
    return torch.device("cuda", 0)


def case_inputs(M, N, K, b, seed, density=0.5, mask=None, bias=False, dy=True):
    R, C = N // b, K // b
    if mask is None:
        mask = synth.uniform_mask(R, C, density, synth.rng(seed, synth.STREAM_PATTERN))
    nnzb = int(mask.sum())
    host = dict(mask=mask, X=synth.activations(M, K, seed), V=synth.block_values(nnzb, b, seed),
                bias=synth.bias_vector(N, seed) if bias else None,
                dY=synth.grad_output(M, N, seed) if dy else None)
    return host


def to_dev(host: dict) -> dict:
    return {k: (v.to(dev()) if isinstance(v, torch.Tensor) else v) for k, v in host.items()}


def check(name: str, g: torch.Tensor, ref: np.ndarray, S: np.ndarray) -> dict:
    res = oracle.tolerance_check(g.cpu(), ref, S)
    say(f"    {name}: max |g-ref|/S = {res['max_ratio']:.3e}, violations {res['violations']} / {res['checked']}")
    assert res["violations"] == 0, f"{name}: {res}"
    return res


def full_parity(M, N, K, b, host: dict, ops=("fwd", "dx", "dw"), dbias=False):
    """Runs the requested ops on the GPU and compares every output element with the oracle."""
    d = to_dev(host)
    p = Pattern.from_mask(host["mask"], N, K, b)
    md = meta.scan(host["mask"])
    out = {}
    if "fwd" in ops:
        Y = binding.linear_fwd(p, d["X"], d["V"], d["bias"])
        torch.cuda.synchronize()
        ref, S = oracle.fwd(host["X"], md["row_ptr"], md["col_idx"], host["V"], N, b, bias=host["bias"])
        out["fwd"] = check("fwd", Y, ref, S)
    if "dx" in ops:
        dX = binding.linear_bwd_input(p, d["dY"], d["V"])
        torch.cuda.synchronize()
        ref, S = oracle.dx(host["dY"], md["row_ptr"], md["col_idx"], host["V"], K, b)
        out["dx"] = check("dx", dX, ref, S)
    if "dw" in ops:
        dV, db = binding.linear_bwd_weight(p, d["dY"], d["X"], want_dbias=dbias)
        torch.cuda.synchronize()
        ref, S = oracle.dw(host["dY"], host["X"], md["row_ptr"], md["col_idx"], b)
        out["dw"] = check("dw", dV, ref, S)
        if dbias:
            ref, S = oracle.db(host["dY"])
            out["db"] = check("db", db, ref, S)
    p.close()
    return out
