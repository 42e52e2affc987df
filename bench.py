#!/usr/bin/env python3
"""Benchmark of the block-sparse linear layer (forward + input grad + weight grad) on one MI355X.

One step = one pass of the whole hot path over one batch: bsr_linear_fwd, then
bsr_linear_bwd_input and bsr_linear_bwd_weight (the ops the workload lists), on seeded
synthetic bf16 inputs already resident in HBM. Useful FLOPs per op are 2*M*b^2*nnzb (work
on zero blocks is never counted).

Headline workload (default): the largest configuration, X[16384,4096] -> Y[16384,11008],
32x32 blocks at overall density 0.3 with Zipf-distributed blocks per block row, fwd + dX +
dW. The headline value is 3F / (time of one step), the step timed over exactly --steps
HIP-graph replays after --warmup eager steps. Buffers are cold: steps rotate over distinct
buffer sets that together hold at least 512 MiB (twice the 256 MB Infinity Cache); one set
of the headline workload is already ~1 GB. --warm reuses one set.

Prints ONE JSON line. Besides the headline: per-op times and the dominant op's roofline,
the same kernels on the density-1.0 pattern of the same shape, hipBLASLt dense
(torch.matmul) as context, the other reference workloads (BERT-base FFN-up, the square
layer at density 0.1, the decode shape) with their own per-op times and rooflines, the
NEXT-row kernels, and the fp64 oracle on the host cores.
"""
from __future__ import annotations

import argparse
import json
import re
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
METRIC = "useful TFLOP/s (2·M·b²·nnzb) fwd+bwd and % bf16 MFMA peak; GB/s at small M"
ROTATE_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def op_bytes(w, nnzb: int, op: str, bias: bool) -> int:
    """Algorithmic bytes of one op: each input read once, each output written once, metadata."""
    M, N, K, b = w.M, w.N, w.K, w.b
    R, C = N // b, K // b
    act_x, act_y, vals = 2 * M * K, 2 * M * N, 2 * nnzb * b * b
    csr = 4 * (R + 1) + 4 * nnzb
    csc = 4 * (C + 1) + 8 * nnzb
    if op == "fwd":
        return act_x + vals + act_y + csr + (2 * N if bias else 0)
    if op == "dx":
        return act_y + vals + act_x + csc
    if op == "dw":
        return act_y + act_x + vals + csr
    raise ValueError(op)


KERNEL_SOURCES = ("sparse_gemm_amd/csrc/bsr_kernels.hip", "sparse_gemm_amd/csrc/bsr_wide.hip",
                  "sparse_gemm_amd/csrc/bsr_device.hpp", "sparse_gemm_amd/csrc/bsr_pattern.cpp",
                  "sparse_gemm_amd/csrc/bsr_internal.hpp")


def op_of_kernel(name: str):
    """The op (fwd, dx, dw) a library kernel belongs to, from its (demangled) name: the panel GEMM
    serves the forward (TRANS false) and the input gradient (TRANS true)."""
    if "bsr" not in name:
        return None
    if "k_panel_gemm" in name:
        # template arguments <BS, G, S, NW, NL, NST, MS, TRANS, SP>: TRANS marks the input gradient,
        # SP other than 0 the 2:4 forward (not part of the step)
        m = re.search(r"k_panel_gemm<([^>]*)>", name)
        args = [a.strip() for a in m.group(1).split(",")] if m else []
        if len(args) >= 9 and args[8] not in ("0", "false"):
            return None
        return "dx" if len(args) >= 8 and args[7] == "true" else "fwd"
    if "k_wide_gemm_24" in name:
        return None   # the 2:4 forward, not part of the step
    if "k_wide_gemm" in name:
        # template argument <TRANS>: the input gradient when true
        return "dx" if "k_wide_gemm<true>" in name else "fwd"
    if "k_small_m" in name:
        return "fwd"
    if any(k in name for k in ("k_dw_panel", "k_dw_reduce", "k_wide_dw", "k_colsum")):
        return "dw"
    return None
COPY_BYTES = 256 << 20   # plain copy used to calibrate the HBM byte counters


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_path(workload_name: str) -> str:
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{workload_name}.txt")


def read_traffic(workload_name: str):
    """HBM bytes per launch of each op from the committed counter summary, or None when the
    summary is missing or was taken with other kernel sources."""
    path = traffic_path(workload_name)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith(("#", " ", "|", "`")):
                k, v = ln.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    out = {}
    for op in ("fwd", "dx", "dw"):
        key = f"{op}_hbm_bytes_per_launch"
        if key in vals:
            out[op] = float(vals[key])
    return out


def summarize_pmc(fetch_dir: str, write_dir: str, workload_name: str, ops, out_path=None) -> str:
    """Per-op HBM bytes per launch from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB
    per dispatch) of `bench.py --calibrate-copy`, each scaled by what the same counter reads for a
    plain copy of COPY_BYTES bytes. Writes the summary under profiles/ and returns its path."""
    import csv
    import glob

    def per_kernel(d, counter):
        rows = {}
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(fn)):
                if r["Counter_Name"] != counter:
                    continue
                rows.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return rows

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")

    def avg(rows, pred):
        v = [x for k, xs in rows.items() if pred(k) for x in xs]
        return sum(v) / len(v) if v else 0.0

    def is_copy(k):
        return "copy" in k.lower() or "elementwise" in k.lower()

    # the calibration copy is the largest copy-like dispatch
    copy_f = max((x for k, xs in fetch.items() if is_copy(k) for x in xs), default=0.0)
    copy_w = max((x for k, xs in write.items() if is_copy(k) for x in xs), default=0.0)
    sf = COPY_BYTES / copy_f if copy_f else 1.0
    sw = COPY_BYTES / copy_w if copy_w else 1.0
    lines = [f"# HBM traffic per launch, {workload_name}", "",
             "Two rocprofv3 counter runs of the benchmark (FETCH_SIZE, then WRITE_SIZE), run from the",
             "repository root on one MI355X:", "",
             "```",
             f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch_dir> -o run -- python3 bench.py "
             f"--workload <k> --steps 3 --warmup 1 --no-cpu-baseline --no-extras --calibrate-copy",
             f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write_dir> -o run -- python3 bench.py "
             f"--workload <k> --steps 3 --warmup 1 --no-cpu-baseline --no-extras --calibrate-copy",
             "python3 bench.py --workload <k> --pmc-summary <fetch_dir> <write_dir>",
             "```", "",
             f"Calibration: a plain copy of {COPY_BYTES} bytes reads FETCH_SIZE = {copy_f:.0f} B and "
             f"WRITE_SIZE = {copy_w:.0f} B;",
             f"kernel bytes below are scaled by {sf:.4f} (reads) and {sw:.4f} (writes).", ""]
    lines.append("| Kernel | dispatches | FETCH B/launch (scaled) | WRITE B/launch (scaled) |")
    lines.append("|---|---|---|---|")
    for k in sorted(set(fetch) | set(write)):
        if "bsr" not in k:
            continue
        f_ = fetch.get(k, [])
        w_ = write.get(k, [])
        short = re.sub(r"\(.*$", "", k.replace("void ", "").replace("bsr::(anonymous namespace)::", ""))
        lines.append(f"| `{short}` | {len(f_)} | {sf * sum(f_) / max(1, len(f_)):.0f} | "
                     f"{sw * sum(w_) / max(1, len(w_)):.0f} |")
    lines.append("")
    lines.append(f"kernel_source_sha256: {kernel_source_hash()}")
    for op in ops:
        # every kernel of the op counts once per launch of the op (e.g. the split-M reduce)
        names = sorted({k for k in set(fetch) | set(write) if op_of_kernel(k) == op})
        per = sum(sf * avg(fetch, lambda k, n=n: k == n) + sw * avg(write, lambda k, n=n: k == n) for n in names)
        lines.append(f"{op}_hbm_bytes_per_launch: {per:.0f}")
    path = out_path or traffic_path(workload_name)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


MFMA_COUNTERS = "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE"
SIMDS = 1024        # 256 compute units x 4 SIMDs
XCCS = 8            # GRBM_GUI_ACTIVE is summed over the 8 XCDs; their counts agree to within a cycle


def mfma_path(workload_name: str) -> str:
    return os.path.join(ROOT, "profiles", f"mfma_counters_{workload_name}.txt")


def summarize_mfma(pmc_dir: str, workload_name: str, seed: int = 0, out_path=None) -> str:
    """Executed bf16 MFMA work and MFMA busy time per library kernel from one rocprofv3 --pmc run
    (MFMA_COUNTERS), against the op's useful flops 2*M*b*b*nnzb. Executed flops = MOPS_BF16 * 512
    (the counter counts multiply and add operations in units of 512); busy = MFMA busy cycles
    summed over the SIMDs / (active cycles x SIMDs). Writes the summary under profiles/."""
    import csv
    import glob
    from sparse_gemm_amd import synth
    w = synth.WORKLOADS[[k for k, x in synth.WORKLOADS.items() if x.name == workload_name][0]]
    nnzb = int(synth.block_mask(w, seed).sum())
    useful = 2.0 * w.M * w.b * w.b * nnzb
    rows = {}
    for fn in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(fn)):
            if "bsr" not in r["Kernel_Name"]:
                continue
            d = rows.setdefault(r["Kernel_Name"], {}).setdefault(r["Dispatch_Id"], {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    lines = [f"# MFMA counters per launch, {workload_name}", "",
             "One rocprofv3 counter run of the benchmark, run from the repository root on one MI355X:", "",
             "```",
             f"rocprofv3 --pmc {MFMA_COUNTERS} --output-format csv -d <dir> -o run -- python3 bench.py "
             "--workload <k> --steps 3 --warmup 1 --no-cpu-baseline --no-extras",
             "python3 bench.py --workload <k> --mfma-summary <dir>",
             "```", "",
             f"Useful flops per op (2*M*b*b*nnzb): {useful:.6e}. Executed = SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512;",
             f"busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {XCCS} * {SIMDS}) over the kernel's run.", "",
             "| Kernel | op | dispatches | executed bf16 MFMA flops / launch | executed / useful | MFMA busy |",
             "|---|---|---|---|---|---|"]
    for k in sorted(rows):
        ds = list(rows[k].values())
        ex = sum(d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for d in ds) / len(ds) * 512.0
        busy = [d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / max(1.0, d.get("GRBM_GUI_ACTIVE", 0.0) / XCCS * SIMDS)
                for d in ds]
        op = op_of_kernel(k)
        ratio = f"{ex / useful:.3f}" if op and ex else "-"
        short = re.sub(r"\(.*$", "", k.replace("void ", "").replace("bsr::(anonymous namespace)::", ""))
        lines.append(f"| `{short}` | {op or '-'} | {len(ds)} | {ex:.6e} | {ratio} | "
                     f"{100.0 * sum(busy) / len(busy):.1f}% |")
    lines.append("")
    lines.append(f"kernel_source_sha256: {kernel_source_hash()}")
    path = out_path or mfma_path(workload_name)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def trace_path(workload_name: str) -> str:
    return os.path.join(ROOT, "profiles", f"kernel_trace_{workload_name}.md")


def summarize_trace(trace_dir: str, workload: int, workload_name: str, out_path=None) -> str:
    """Per-kernel durations from one rocprofv3 --kernel-trace --stats run of the benchmark
    (its *kernel_stats.csv). Writes the summary under profiles/ and returns its path."""
    import csv
    import glob
    src = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True))
    if not src:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = list(csv.DictReader(open(src[0])))
    tot = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    lines = [f"# Kernel trace: bench.py, workload {workload_name}", "",
             "Commands (run from the repository root on one MI355X):", "", "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- python3 bench.py "
             f"--workload {workload} --steps 20 --warmup 5 --no-cpu-baseline --no-extras",
             f"python3 bench.py --workload {workload} --trace-summary <dir>", "```", "",
             "| Kernel | Calls | Avg (us) | Min (us) | Max (us) | % of GPU time |", "|---|---|---|---|---|---|"]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    for r in rows:
        short = re.sub(r"\(.*$", "", r["Name"].replace("void ", "").replace("bsr::(anonymous namespace)::", "")
                       .replace("(anonymous namespace)::", ""))
        if len(short) > 100:
            short = short[:97] + "..."
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{100 * float(r['TotalDurationNs']) / tot:.2f} |")
    lines.append("")
    lines.append(f"kernel_source_sha256: {kernel_source_hash()}")
    path = out_path or trace_path(workload_name)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _sleep_cycles_per_ms() -> float:
    """Rate of the spin kernel torch.cuda._sleep, measured with HIP events."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    a.record()
    torch.cuda._sleep(2_000_000)
    b.record()
    torch.cuda.synchronize()
    return 2_000_000 / max(1e-3, a.elapsed_time(b))


def time_ops(run_step, nsteps: int, warmup: int, ops, hold_ms: float):
    """Per-op GPU durations with HIP events on the launch stream (torch's current stream).

    A spin kernel holds the GPU while the host enqueues all timed steps, so back-to-back
    kernels run with no host gaps and each event pair brackets GPU execution plus the
    dispatch of the op's first kernel. Returns (GPU ms per step, {op: avg ms},
    {op: (p10, median, p90) ms}, host enqueue s)."""
    import torch
    for k in range(warmup):
        run_step(k, None)
    torch.cuda.synchronize()
    evs = {op: [] for op in ops}
    first, last = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(hold_ms * _CYC_PER_MS))
    first.record()
    t = time.perf_counter()
    for k in range(nsteps):
        run_step(warmup + k, evs)
    last.record()
    enqueue_s = time.perf_counter() - t
    torch.cuda.synchronize()
    step_ms = first.elapsed_time(last) / nsteps
    op_ms, pct = {}, {}
    for op in ops:
        ts = sorted(a.elapsed_time(b) for a, b in evs[op])
        op_ms[op] = sum(ts) / max(1, len(ts))
        if ts:
            q = lambda f: ts[min(len(ts) - 1, int(round(f * (len(ts) - 1))))]
            pct[op] = (q(0.1), q(0.5), q(0.9))
    if enqueue_s * 1e3 > hold_ms:
        log(f"[bench] warning: host enqueue took {enqueue_s * 1e3:.1f} ms > hold {hold_ms:.1f} ms; "
            "op times may include host gaps")
    return step_ms, op_ms, pct, enqueue_s


def time_graph_steps(run_step, nsets: int, nsteps: int, hold_ms: float = 20.0):
    """Exactly `nsteps` timed steps: one HIP graph holding steps 0 .. nsteps-1 (step k on buffer
    set k % nsets), captured after an eager pass on the capture stream and replayed once untimed,
    then replayed once between two synchronizes with HIP events and the wall clock around it.
    Returns (event ms per step, wall ms per step)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for k in range(min(nsets, nsteps)):
            run_step(k, None)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(nsteps):
            run_step(k, None)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(hold_ms * _CYC_PER_MS))
    t = time.perf_counter()
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t
    del g
    return a.elapsed_time(b) / nsteps, wall / nsteps * 1e3


_CYC_PER_MS = 1.0


def set_bytes(w, nnzb: int) -> int:
    """Distinct bytes of one buffer set: every tensor the step reads or writes, once."""
    b2 = 2 * nnzb * w.b * w.b
    by = 2 * w.M * w.K + b2 + 2 * w.M * w.N + (2 * w.N if w.bias else 0)
    if "dx" in w.ops or "dw" in w.ops:
        by += 2 * w.M * w.N
    if "dx" in w.ops:
        by += 2 * w.M * w.K
    if "dw" in w.ops:
        by += b2
    return by


def rotation_sets(w, nnzb: int, warm: bool) -> int:
    return 1 if warm else max(1, -(-ROTATE_BYTES // max(1, set_bytes(w, nnzb))))


def build_sets(w, host, nsets: int, dev, share=None):
    """nsets buffer sets on the device. With `share` (sets of another pattern of the same shape),
    only the block values and their gradient are new; activations and outputs are reused."""
    import torch
    sets = []
    for k in range(nsets):
        s = {}
        if share is not None:
            s.update({key: share[k % len(share)][key] for key in ("X", "dY", "bias", "Y", "dX") if key in share[0]})
        else:
            for key in ("X", "dY"):
                if host.get(key) is not None:
                    s[key] = host[key].to(dev) if k == 0 else sets[0][key].clone()
            s["bias"] = host["bias"].to(dev) if host.get("bias") is not None else None
            s["Y"] = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
            if "dx" in w.ops:
                s["dX"] = torch.empty((w.M, w.K), dtype=torch.bfloat16, device=dev)
        s["V"] = host["V"].to(dev) if k == 0 else sets[0]["V"].clone()
        if "dw" in w.ops:
            s["dV"] = torch.empty_like(s["V"])
        sets.append(s)
    return sets


def make_runner(p, w, sets, ws, only=None):
    import torch
    from sparse_gemm_amd import binding

    def run_step(k, evs):
        s = sets[k % len(sets)]
        for op in (w.ops if only is None else (only,)):
            if evs is not None:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
            if op == "fwd":
                binding.linear_fwd(p, s["X"], s["V"], s["bias"], out=s["Y"])
            elif op == "dx":
                binding.linear_bwd_input(p, s["dY"], s["V"], out=s["dX"])
            elif op == "dw":
                binding.linear_bwd_weight(p, s["dY"], s["X"], out=s["dV"], workspace=ws)
            if evs is not None:
                b.record()
                evs[op].append((a, b))
    return run_step


def time_launches(fn, nsets: int, reps: int) -> float:
    """Average ms per launch of fn(k) over reps launches cycling nsets buffer sets, HIP events
    on the launch stream with the queue pre-filled behind a spin kernel."""
    import torch
    for k in range(min(3, reps)):
        fn(k)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(20.0 * _CYC_PER_MS))
    a.record()
    for k in range(reps):
        fn(k)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def op_kernels(p, w, op: str):
    """Library kernels one launch of the op runs at this workload, as the library dispatches them."""
    from sparse_gemm_amd import binding
    return binding.op_kernels(p, op, w.M)


def roofline_of(w, nnzb: int, op: str, t_s: float, traffic) -> dict:
    F = 2.0 * w.M * w.b * w.b * nnzb
    by = op_bytes(w, nnzb, op, w.bias)
    if F / by < RIDGE:
        r = {"bound": "hbm", "achieved": by / t_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        r = {"bound": "mfma", "achieved": F / t_s / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    r["frac"] = r["achieved"] / r["peak"]
    r["traffic"] = traffic
    return r


def measure(w, host, dev, nsteps: int, warmup: int, warm: bool, extras: bool, label: str) -> dict:
    """One workload: the whole step (fwd [+ dX + dW]) over rotated cold buffer sets, per-op
    times, the dominant op's roofline, a cache-warm step, and (extras) the same kernels at
    density 1.0 and hipBLASLt dense GEMMs of the same shapes."""
    import numpy as np
    import torch
    from sparse_gemm_amd import binding, synth
    mask = host["mask"]
    nnzb = int(mask.sum())
    p = binding.Pattern.from_mask(mask, w.N, w.K, w.b)
    F = 2.0 * w.M * w.b * w.b * nnzb
    nsets = rotation_sets(w, nnzb, warm)
    sets = build_sets(w, host, nsets, dev)
    ws_bytes = binding.bwd_weight_workspace_bytes(p, w.M) if "dw" in w.ops else 0
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev) if ws_bytes else None
    dist = set_bytes(w, nnzb)
    log(f"[bench] {label}: {w.name}, nnzb {nnzb}, {nsets} buffer set(s) of {dist / 1e6:.1f} MB")
    run = make_runner(p, w, sets, ws)
    eager_ms, op_in_step, pct, enq = time_ops(run, nsteps, warmup, w.ops, hold_ms=50.0 + 2.0 * nsteps)
    step_ms, wall_ms = time_graph_steps(run, nsets, nsteps)
    nops = len(w.ops)
    # each op alone, launched back to back over the rotated sets: the kernels' own durations
    op_alone = {op: time_launches(lambda k, r=make_runner(p, w, sets, ws, only=op): r(k, None), nsets,
                                  max(20, nsteps)) for op in w.ops}
    log(f"[bench] {label}: step {step_ms * 1e3:.1f} us (graph), " +
        ", ".join(f"{o} {t * 1e3:.1f} us" for o, t in op_alone.items()))
    tr = read_traffic(w.name)
    per_op = {}
    for op in w.ops:
        t = op_alone[op] * 1e-3
        by = op_bytes(w, nnzb, op, w.bias)
        t_roof = max(F / (PEAK_BF16_TFLOPS * 1e12), by / (PEAK_HBM_GBS * 1e9))
        per_op[op] = {"us": op_alone[op] * 1e3, "us_in_step": op_in_step[op] * 1e3,
                      "tflops": F / t / 1e12, "pct_mfma_peak": 100 * F / t / 1e12 / PEAK_BF16_TFLOPS,
                      "gbs": by / t / 1e9, "pct_hbm_peak": 100 * by / t / 1e9 / PEAK_HBM_GBS, "bytes": by,
                      "pct_roofline": 100 * t_roof / t, "kernels": op_kernels(p, w, op)}
        if op in pct:
            per_op[op].update({"p10_us_in_step": pct[op][0] * 1e3, "median_us_in_step": pct[op][1] * 1e3,
                               "p90_us_in_step": pct[op][2] * 1e3})
    dom = max(w.ops, key=lambda o: op_alone[o])
    roof = roofline_of(w, nnzb, dom, op_alone[dom] * 1e-3, tr.get(dom) if tr else None)
    roof["kernel"] = {"fwd": "bsr_linear_fwd", "dx": "bsr_linear_bwd_input", "dw": "bsr_linear_bwd_weight"}[dom]
    roof["per_launch"] = {"flops": F, "algorithmic_bytes": op_bytes(w, nnzb, dom, w.bias),
                          "avg_us": op_alone[dom] * 1e3, "kernels": op_kernels(p, w, dom),
                          "timing": "back-to-back launches over the rotated buffer sets, HIP events on the "
                                    "launch stream, queue pre-filled behind a spin kernel"}
    res = {"workload": w.name, "M": w.M, "K": w.K, "N": w.N, "block": w.b, "density": w.density, "nnzb": nnzb,
           "pattern": w.pattern, "ops": "+".join(w.ops),
           "buffers": (f"cold ({nsets} rotated sets of {dist} distinct bytes, {nsets * dist} in all)" if not warm
                       else "warm (1 set)"),
           "rotated_bytes": nsets * dist,
           "pattern_sha256": synth.mask_digest(mask), "rows": synth.row_histogram(mask),
           "ms_per_step": step_ms, "steps": nsteps,
           "tflops": nops * F / (step_ms * 1e-3) / 1e12,
           "pct_bf16_mfma_peak": 100 * nops * F / (step_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "ops": per_op, "roofline": roof,
           "timing": {"ms_per_step": "one HIP graph of exactly `steps` steps (buffer sets in rotation) replayed "
                                     "between two synchronizes, HIP events",
                      "graph_wall_ms_per_step": wall_ms, "eager_gpu_ms_per_step": eager_ms,
                      "eager_host_enqueue_ms_per_step": enq * 1e3 / nsteps,
                      "ops.us": "each op alone, back-to-back launches over the rotated sets (kernel durations)",
                      "ops.us_in_step": "HIP events around each call inside eager steps (includes the "
                                        "dispatch of the op's first kernel)"}}
    if not warm and nsets > 1:
        res["warm_ms_per_step"], _ = time_graph_steps(make_runner(p, w, sets[:1], ws), 1, nsteps)
    elif not warm:
        res["warm_ms_per_step"] = None   # one set already exceeds the rotation size: no warm variant
    if extras:
        # the same kernels on the density-1.0 pattern of the same shape (activations shared)
        full = np.ones_like(mask)
        host_d = {"mask": full, "V": synth.block_values(int(full.sum()), w.b, 0)}
        pd = binding.Pattern.from_mask(full, w.N, w.K, w.b)
        nnzd = int(full.sum())
        nsets_d = min(nsets, rotation_sets(w, nnzd, warm))
        sets_d = build_sets(w, host_d, nsets_d, dev, share=sets)
        wsd_b = binding.bwd_weight_workspace_bytes(pd, w.M) if "dw" in w.ops else 0
        wsd = torch.empty((wsd_b,), dtype=torch.uint8, device=dev) if wsd_b else None
        run_d = make_runner(pd, w, sets_d, wsd)
        nd = max(10, nsteps // 2)
        for k in range(3):
            run_d(k, None)
        d_ms, _ = time_graph_steps(run_d, nsets_d, nd)
        d_alone = {op: time_launches(lambda k, r=make_runner(pd, w, sets_d, wsd, only=op): r(k, None), nsets_d, nd)
                   for op in w.ops}
        res["density_1.0_same_kernels"] = {
            "ms_per_step": d_ms, "speedup_of_sparse": d_ms / step_ms,
            "ops_us": {o: t * 1e3 for o, t in d_alone.items()},
            "ops_speedup_of_sparse": {o: d_alone[o] / op_alone[o] for o in w.ops},
            "tflops": nops * 2.0 * w.M * w.b * w.b * nnzd / (d_ms * 1e-3) / 1e12,
            "buffers": f"{nsets_d} rotated set(s)"}
        log(f"[bench] {label}: density 1.0 step {d_ms * 1e3:.1f} us ({d_ms / step_ms:.2f}x the sparse step)")
        del sets_d, wsd
        pd.close()
        # hipBLASLt dense GEMMs of the same shapes (torch.matmul; context only)
        dense_w = [s_["V"].new_empty((w.N, w.K)).normal_() for s_ in sets[:max(1, min(nsets, 2))]]

        def dense_step(k, evs):
            s_ = sets[k % len(dense_w)]
            Wd = dense_w[k % len(dense_w)]
            torch.matmul(s_["X"], Wd.t(), out=s_["Y"])
            if "dx" in w.ops:
                torch.matmul(s_["dY"], Wd, out=s_["dX"])
            if "dw" in w.ops:
                torch.matmul(s_["dY"].t(), s_["X"])
        for k in range(3):
            dense_step(k, None)
        h_ms, _ = time_graph_steps(dense_step, len(dense_w), max(10, nsteps // 2))
        res["hipblaslt_dense_context"] = {"ms_per_step": h_ms, "speedup_of_sparse": h_ms / step_ms,
                                          "dense_tflops": nops * 2.0 * w.M * w.N * w.K / (h_ms * 1e-3) / 1e12}
        del dense_w
    del sets, ws
    p.close()
    return res


def cpu_baseline(w, host, seconds: float) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the same workload (the first rows of
    X and dY, the whole pattern) on the host's cores: each op gets about seconds / ops of wall
    time. Threads: the cores this process may run on, capped by OMP_NUM_THREADS when set."""
    import oracle
    from oracle import meta
    threads = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        threads = min(threads, int(env))
    oracle.set_threads(threads)
    md = meta.scan(host["mask"])
    nnzb = md["nnzb"]
    F_row = 2.0 * w.b * w.b * nnzb        # useful flops per activation row and op
    X64 = oracle._f64(host["X"])
    dY64 = oracle._f64(host["dY"]) if host.get("dY") is not None else None
    budget = seconds / len(w.ops)
    ops = {}
    tot_f = tot_t = 0.0
    for op in w.ops:
        probe = min(w.M, 32)
        t = time.perf_counter()
        _run_oracle(w, md, host, X64, dY64, probe, op)
        per_row = max(1e-6, (time.perf_counter() - t) / probe)
        rows = int(min(w.M, max(probe, budget / per_row)))
        reps = max(1, int(round(budget / (per_row * rows)))) if rows == w.M else 1
        t = time.perf_counter()
        for _ in range(reps):
            _run_oracle(w, md, host, X64, dY64, rows, op)
        dt = time.perf_counter() - t
        f = F_row * rows * reps
        ops[op] = {"rows": rows, "reps": reps, "wall_s": dt, "gflops": f / dt / 1e9,
                   "ms_full_workload": dt / (rows * reps) * w.M * 1e3}
        tot_f += f
        tot_t += dt
    return {"value": tot_f / tot_t / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": (f"the first rows of {w.M} (per op: " +
                       ", ".join(f"{o} {v['rows']} rows x {v['reps']}" for o, v in ops.items()) +
                       f") of the workload with its whole pattern, fp64, no tolerance sums, {tot_t:.1f} s wall"),
            "ops": ops, "cpu_model": cpu_model(), "seconds": tot_t}


def _run_oracle(w, md, host, X64, dY64, rows, op):
    import oracle
    if op == "fwd":
        oracle.fwd(X64[:rows], md["row_ptr"], md["col_idx"], host["V"], w.N, w.b, bias=host["bias"], want_s=False)
    elif op == "dx":
        oracle.dx(dY64[:rows], md["row_ptr"], md["col_idx"], host["V"], w.K, w.b, want_s=False)
    elif op == "dw":
        oracle.dw(dY64[:rows], X64[:rows], md["row_ptr"], md["col_idx"], w.b, want_s=False)


CONVERT_WORKLOAD = 5   # the largest weight of the reference workloads: 11008 x 4096, Zipf rows


def convert_leg(dev, reps: int) -> dict:
    """Dense <-> BSR conversion and block magnitudes (bsr_block_norms, bsr_dense_to_values,
    bsr_values_to_dense) on the weight of the Zipf workload, cold (rotated sets), with their
    algorithmic bytes and the fraction of HBM peak."""
    import torch
    from sparse_gemm_amd import binding, synth
    w = synth.WORKLOADS[CONVERT_WORKLOAD]
    mask = synth.block_mask(w, 0)
    p = binding.Pattern.from_mask(mask, w.N, w.K, w.b)
    nnzb, R, C, b = p.nnzb, w.R, w.C, w.b
    dense_bytes = 2 * w.N * w.K
    nsets = max(1, -(-ROTATE_BYTES // dense_bytes))
    W0 = synth.dense_weight(w.N, w.K, 0, b=b).to(dev)
    Ws = [W0] + [W0.clone() for _ in range(nsets - 1)]
    Vs = [torch.empty((nnzb, b, b), dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
    Ns = [torch.empty((R, C), dtype=torch.float64, device=dev) for _ in range(nsets)]
    Ds = [torch.empty((w.N, w.K), dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
    csr = 4 * (R + 1) + 4 * nnzb
    legs = {
        "block_norms_l1": (lambda k: binding.block_norms(Ws[k % nsets], b, 1, out=Ns[k % nsets]),
                           dense_bytes + 8 * R * C),
        "dense_to_values": (lambda k: binding.dense_to_values(p, Ws[k % nsets], out=Vs[k % nsets]),
                            2 * 2 * b * b * nnzb + csr),
        "values_to_dense": (lambda k: binding.values_to_dense(p, Vs[k % nsets], out=Ds[k % nsets]),
                            2 * b * b * nnzb + dense_bytes + csr),
    }
    out = {"weight": f"{w.N}x{w.K}, b {b}, nnzb {nnzb} ({w.pattern} rows, density {w.density})",
           "buffers": f"cold ({nsets} rotated sets)"}
    for name, (fn, by) in legs.items():
        ms = time_launches(fn, nsets, reps)
        out[name] = {"us": ms * 1e3, "bytes": by, "gbs": by / (ms * 1e-3) / 1e9,
                     "pct_hbm_peak": 100 * by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del Ws, Vs, Ns, Ds
    p.close()
    return out


FP8_WORKLOAD = 4   # the memory-bound decode shape: X[8,4096], W[14336,4096], 64 x 64 blocks


def fp8_leg(dev, reps: int) -> dict:
    """The decode forward with fp8 (E4M3) block values and a power-of-two scale per block
    (bsr_linear_fwd_fp8) beside the bf16 forward (bsr_linear_fwd) on the same pattern, cold
    (rotated value sets), with algorithmic bytes and the fraction of HBM peak."""
    import torch
    from sparse_gemm_amd import binding, synth
    w = synth.WORKLOADS[FP8_WORKLOAD]
    host = synth.make_inputs(w, 0)
    p = binding.Pattern.from_mask(host["mask"], w.N, w.K, w.b)
    nnzb, R = p.nnzb, w.R
    X = host["X"].to(dev)
    Y = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
    V0 = host["V"].to(dev)
    code_bytes = nnzb * w.b * w.b
    nsets = max(1, -(-ROTATE_BYTES // code_bytes))
    q = [binding.values_quantize_fp8(p, V0)]
    q += [(a.clone(), s_.clone()) for a, s_ in [q[0]] * (nsets - 1)]
    nsets16 = max(1, -(-ROTATE_BYTES // (2 * code_bytes)))
    V16 = [V0] + [V0.clone() for _ in range(nsets16 - 1)]
    meta = 4 * (R + 1) + 4 * nnzb
    act = 2 * w.M * w.K + 2 * w.M * w.N
    by8 = code_bytes + 4 * nnzb + act + meta
    by16 = 2 * code_bytes + act + meta
    ms8 = time_launches(lambda k: binding.linear_fwd_fp8(p, X, q[k % nsets][0], q[k % nsets][1], out=Y), nsets, reps)
    ms16 = time_launches(lambda k: binding.linear_fwd(p, X, V16[k % nsets16], out=Y), nsets16, reps)
    F = 2.0 * w.M * w.b * w.b * nnzb
    out = {"workload": w.name, "buffers": f"cold ({nsets} rotated fp8 value sets, {nsets16} bf16)",
           "fwd_fp8": {"us": ms8 * 1e3, "bytes": by8, "gbs": by8 / (ms8 * 1e-3) / 1e9,
                       "pct_hbm_peak": 100 * by8 / (ms8 * 1e-3) / 1e9 / PEAK_HBM_GBS,
                       "tflops": F / (ms8 * 1e-3) / 1e12},
           "fwd_bf16": {"us": ms16 * 1e3, "bytes": by16, "gbs": by16 / (ms16 * 1e-3) / 1e9,
                        "pct_hbm_peak": 100 * by16 / (ms16 * 1e-3) / 1e9 / PEAK_HBM_GBS},
           "speedup_fp8_vs_bf16": ms16 / ms8}
    del q, V16
    p.close()
    return out


def sparse24_leg(dev, reps: int) -> dict:
    """The decode forward with 2:4 sparsity inside every kept block (bsr_linear_fwd_24, sparse
    matrix cores) on the decode workload's pattern, its blocks pruned to 2:4, cold (rotated value
    sets); algorithmic bytes: compressed values + indices + activations + CSR."""
    import torch
    from sparse_gemm_amd import binding, synth
    w = synth.WORKLOADS[FP8_WORKLOAD]
    host = synth.make_inputs(w, 0)
    p = binding.Pattern.from_mask(host["mask"], w.N, w.K, w.b)
    nnzb, R = p.nnzb, w.R
    X = host["X"].to(dev)
    Y = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
    c0 = binding.values_compress_24(p, host["V"].to(dev))
    vc_bytes = nnzb * w.b * w.b
    meta_bytes = nnzb * w.b * (w.b // 16) * 2
    nsets = max(1, -(-ROTATE_BYTES // (vc_bytes + meta_bytes)))
    cs = [c0] + [(a.clone(), m.clone()) for a, m in [c0] * (nsets - 1)]
    by = vc_bytes + meta_bytes + 2 * w.M * w.K + 2 * w.M * w.N + 4 * (R + 1) + 4 * nnzb
    ms = time_launches(lambda k: binding.linear_fwd_24(p, X, cs[k % nsets][0], cs[k % nsets][1], out=Y), nsets, reps)
    F_kept = 2.0 * w.M * (w.b * w.b // 2) * nnzb
    out = {"workload": w.name + " (blocks pruned to 2:4)", "buffers": f"cold ({nsets} rotated sets)",
           "fwd_24": {"us": ms * 1e3, "bytes": by, "gbs": by / (ms * 1e-3) / 1e9,
                      "pct_hbm_peak": 100 * by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      "tflops_on_kept_values": F_kept / (ms * 1e-3) / 1e12}}
    del cs
    # the kept values as fp8 codes with a power-of-two scale per block (bsr_linear_fwd_fp8_24)
    q0 = binding.values_quantize_fp8_24(p, c0[0])
    by8 = vc_bytes // 2 + 4 * nnzb + meta_bytes + 2 * w.M * w.K + 2 * w.M * w.N + 4 * (R + 1) + 4 * nnzb
    nsets8 = max(1, -(-ROTATE_BYTES // (vc_bytes // 2 + meta_bytes)))
    qs = [(q0[0], q0[1], c0[1])] + [(q0[0].clone(), q0[1].clone(), c0[1].clone()) for _ in range(nsets8 - 1)]
    ms8 = time_launches(lambda k: binding.linear_fwd_fp8_24(p, X, *qs[k % nsets8], out=Y), nsets8, reps)
    out["fwd_fp8_24"] = {"us": ms8 * 1e3, "bytes": by8, "gbs": by8 / (ms8 * 1e-3) / 1e9,
                         "pct_hbm_peak": 100 * by8 / (ms8 * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "buffers": f"cold ({nsets8} rotated sets)"}
    del qs
    p.close()
    return out


SPARSE24_LARGE_WORKLOAD = 5   # the matrix-core-bound Zipf layer


def sparse24_large_leg(dev, reps: int) -> dict:
    """The large-M forward with 2:4 blocks on the sparse matrix cores, from the compressed form
    (bsr_linear_fwd_24: the wide tile staging 1 KB of kept values and 128 B of index words per block)
    and from block images (bsr_linear_fwd_24_image), beside the bf16 forward on the same pattern (the
    Zipf workload, its blocks pruned to 2:4; one buffer set, which already touches ~0.5 GB per
    launch). Useful FLOPs of the 2:4 forward count the kept half of every block."""
    import torch
    from sparse_gemm_amd import binding, synth
    w = synth.WORKLOADS[SPARSE24_LARGE_WORKLOAD]
    host = synth.make_inputs(w, 0, with_dy=False)
    p = binding.Pattern.from_mask(host["mask"], w.N, w.K, w.b)
    X, V = host["X"].to(dev), host["V"].to(dev)
    Y = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
    Vc, mt = binding.values_compress_24(p, V)
    img = binding.values_pack_24(p, Vc, mt)
    ms16 = time_launches(lambda k: binding.linear_fwd(p, X, V, out=Y), 1, reps)
    msc = time_launches(lambda k: binding.linear_fwd_24(p, X, Vc, mt, out=Y), 1, reps)
    ms24 = time_launches(lambda k: binding.linear_fwd_24_image(p, X, img, out=Y), 1, reps)
    F = 2.0 * w.M * w.b * w.b * p.nnzb
    out = {"workload": w.name + " (blocks pruned to 2:4)", "kernel": binding.op_kernels(p, "fwd_24", w.M),
           "fwd_24_us": msc * 1e3, "fwd_24_image_us": ms24 * 1e3, "fwd_bf16_us": ms16 * 1e3,
           "tflops_on_kept_values": F / 2 / (msc * 1e-3) / 1e12,
           "bf16_tflops": F / (ms16 * 1e-3) / 1e12, "speedup_vs_bf16": ms16 / msc,
           "image_speedup_vs_bf16": ms16 / ms24}
    del X, V, Y, Vc, mt, img
    p.close()
    return out


def rebuild_leg(dev, reps: int) -> dict:
    """The on-device metadata rebuild (bsr_meta_rebuild: six small kernels) on the Zipf workload's
    block mask (344 x 128)."""
    import torch
    from sparse_gemm_amd import binding, synth
    w = synth.WORKLOADS[CONVERT_WORKLOAD]
    mask = torch.from_numpy(synth.block_mask(w, 0)).to(dev)
    out = binding.meta_rebuild(mask)
    R, C = mask.shape
    ws = out["_workspace"]
    L = binding.lib()
    st = torch.cuda.current_stream(dev).cuda_stream

    def run(k):
        L.bsr_meta_rebuild(R, C, mask.data_ptr(), out["row_ptr"].data_ptr(), out["col_idx"].data_ptr(),
                           out["col_ptr"].data_ptr(), out["row_idx"].data_ptr(), out["perm"].data_ptr(), R * C,
                           out["nnzb"].data_ptr(), ws.data_ptr(), ws.numel(), st)
    ms = time_launches(run, 1, reps)
    return {"grid": f"{R}x{C}", "nnzb": int(out["nnzb"].item()), "us_per_rebuild": ms * 1e3, "kernels": 6}


HEADLINE_WORKLOAD = 5   # the largest configuration: 16384 x 4096 -> 11008, Zipf rows, fwd + dX + dW
OTHER_WORKLOADS = (2, 3, 4)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=HEADLINE_WORKLOAD,
                    help=f"reference workload 1..5 of the headline line (default {HEADLINE_WORKLOAD})")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--warm", action="store_true", help="reuse one buffer set (cache-warm)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline workload: no density-1.0, hipBLASLt, other-workload or NEXT legs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help=f"also run one plain {COPY_BYTES}-byte device copy (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarize two rocprofv3 --pmc runs into profiles/ and exit (no GPU needed)")
    ap.add_argument("--mfma-summary", metavar="PMC_DIR",
                    help="summarize one rocprofv3 --pmc run of the MFMA counters into profiles/ and exit")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="summarize one rocprofv3 --kernel-trace --stats run into profiles/ and exit")
    args = ap.parse_args()

    if args.trace_summary:
        from sparse_gemm_amd import synth
        print(summarize_trace(args.trace_summary, args.workload, synth.WORKLOADS[args.workload].name))
        return

    if args.mfma_summary:
        from sparse_gemm_amd import synth
        print(summarize_mfma(args.mfma_summary, synth.WORKLOADS[args.workload].name, args.seed))
        return
    if args.pmc_summary:
        from sparse_gemm_amd import synth
        w = synth.WORKLOADS[args.workload]
        print(summarize_pmc(args.pmc_summary[0], args.pmc_summary[1], w.name, w.ops))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_gemm_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    global _CYC_PER_MS
    _CYC_PER_MS = _sleep_cycles_per_ms()
    extras = not args.no_extras

    w = synth.WORKLOADS[args.workload]
    log(f"[bench] headline workload {w.name}; generating inputs")
    host = synth.make_inputs(w, args.seed)
    head = measure(w, host, dev, args.steps, args.warmup, args.warm, extras, "headline")
    small = "dx" not in w.ops and "dw" not in w.ops and w.M <= 64
    if small:
        # memory-bound decode shape: the metric is HBM GB/s of the forward
        by = op_bytes(w, head["nnzb"], "fwd", w.bias)
        value, unit = by / (head["ms_per_step"] * 1e-3) / 1e9, "GB/s"
    else:
        value, unit = head["tflops"], "TFLOP/s"
    out = {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) activations and output gradients, N(0,0.02) blocks)",
           "config": {k: head[k] for k in ("workload", "M", "K", "N", "block", "density", "nnzb", "pattern", "ops",
                                           "buffers", "rotated_bytes", "pattern_sha256", "rows")},
           "pct_bf16_mfma_peak": head["pct_bf16_mfma_peak"],
           "ops": head["ops"], "roofline": head["roofline"], "timing": head["timing"],
           "warm_ms_per_step": head.get("warm_ms_per_step")}
    for k in ("density_1.0_same_kernels", "hipblaslt_dense_context"):
        if k in head:
            out[k] = head[k]

    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host cores")
        out["cpu_baseline"] = cpu_baseline(w, host, args.cpu_seconds)
    del host

    if extras:
        out["other_workloads"] = {}
        for k in OTHER_WORKLOADS:
            if k == args.workload:
                continue
            wk = synth.WORKLOADS[k]
            log(f"[bench] workload {wk.name}; generating inputs")
            hk = synth.make_inputs(wk, args.seed)
            r = measure(wk, hk, dev, args.steps, args.warmup, args.warm, True, f"workload {k}")
            if "dx" not in wk.ops:
                by = op_bytes(wk, r["nnzb"], "fwd", wk.bias)
                r["gbs_per_step"] = by / (r["ms_per_step"] * 1e-3) / 1e9
                r["pct_hbm_peak_per_step"] = 100 * r["gbs_per_step"] / PEAK_HBM_GBS
            out["other_workloads"][wk.name] = r
            del hk
        log("[bench] dense <-> BSR conversion kernels")
        out["next_rows"] = {"convert": convert_leg(dev, max(20, args.steps))}
        log("[bench] fp8 block values, decode forward")
        out["next_rows"]["fp8_decode"] = fp8_leg(dev, max(50, args.steps))
        log("[bench] 2:4 inside blocks, large-M forward")
        out["next_rows"]["sparse24_large"] = sparse24_large_leg(dev, max(10, args.steps // 2))
        log("[bench] on-device metadata rebuild")
        out["next_rows"]["meta_rebuild"] = rebuild_leg(dev, max(50, args.steps))
        log("[bench] 2:4 inside blocks, decode forward")
        out["next_rows"]["sparse24_decode"] = sparse24_leg(dev, max(50, args.steps))
        out["next_rows"]["sparse24_decode"]["speedup_vs_bf16_dense_blocks"] = (
            out["next_rows"]["fp8_decode"]["fwd_bf16"]["us"] / out["next_rows"]["sparse24_decode"]["fwd_24"]["us"])

    if args.calibrate_copy:
        src = torch.empty((COPY_BYTES,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
