"""Host logic of bench.py (no GPU): which op a library kernel belongs to, and the arithmetic of the
rocprofv3 counter summaries (calibration scaling of the byte counters, executed MFMA flops and busy
fraction), on small counter files written here."""
import csv
import os

import bench
from sparse_gemm_amd import synth

PREFIX = "void bsr::(anonymous namespace)::"


def test_op_of_kernel():
    pg = PREFIX + "k_panel_gemm<32, {g}, {s}, 4, 4, 2, 1, {t}, {sp}>(unsigned short const*, int)"
    assert bench.op_of_kernel(pg.format(g=2, s=4, t="false", sp="false")) == "fwd"
    assert bench.op_of_kernel(pg.format(g=1, s=2, t="true", sp="false")) == "dx"
    assert bench.op_of_kernel(pg.format(g=2, s=4, t="false", sp="true")) is None   # 2:4 forward
    assert bench.op_of_kernel(pg.format(g=2, s=4, t="false", sp=0)) == "fwd"
    assert bench.op_of_kernel(pg.format(g=2, s=4, t="true", sp=0)) == "dx"
    assert bench.op_of_kernel(pg.format(g=2, s=4, t="false", sp=1)) is None        # 2:4 images
    assert bench.op_of_kernel(pg.format(g=2, s=4, t="false", sp=2)) is None        # compressed 2:4
    assert bench.op_of_kernel(PREFIX + "k_wide_gemm<false>(bsr::WideArgs)") == "fwd"
    assert bench.op_of_kernel(PREFIX + "k_wide_gemm<true>(bsr::WideArgs)") == "dx"
    assert bench.op_of_kernel(PREFIX + "k_wide_gemm_24(bsr::WideArgs24)") is None
    assert bench.op_of_kernel(PREFIX + "k_small_m<64, 8, 1, 2, true, false, true>(unsigned short const*)") == "fwd"
    assert bench.op_of_kernel(PREFIX + "k_dw_panel<32, 2>(unsigned short const*)") == "dw"
    assert bench.op_of_kernel(PREFIX + "k_dw_reduce(float const*, int, unsigned long, unsigned short*)") == "dw"
    assert bench.op_of_kernel("__amd_rocclr_copyBuffer") is None


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path):
    fwd = PREFIX + "k_panel_gemm<32, 2, 4, 4, 4, 2, 1, false, false>(unsigned short const*)"
    # the copy of COPY_BYTES reads half of them by the counter: reads scale by 2, writes by 1
    half_kib = bench.COPY_BYTES / 2 / 1024
    _write(str(tmp_path / "f" / "run_counter_collection.csv"), [
        {"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE", "Counter_Value": half_kib},
        {"Dispatch_Id": 2, "Kernel_Name": fwd, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1000.0},
        {"Dispatch_Id": 3, "Kernel_Name": fwd, "Counter_Name": "FETCH_SIZE", "Counter_Value": 3000.0}])
    _write(str(tmp_path / "w" / "run_counter_collection.csv"), [
        {"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE",
         "Counter_Value": bench.COPY_BYTES / 1024},
        {"Dispatch_Id": 2, "Kernel_Name": fwd, "Counter_Name": "WRITE_SIZE", "Counter_Value": 500.0},
        {"Dispatch_Id": 3, "Kernel_Name": fwd, "Counter_Name": "WRITE_SIZE", "Counter_Value": 500.0}])
    out = str(tmp_path / "traffic.txt")
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "w", ("fwd",), out_path=out)
    vals = dict(ln.split(":", 1) for ln in open(out) if ln.startswith("fwd_hbm"))
    # average fetch 2000 KiB x 2 + average write 500 KiB x 1
    assert float(vals["fwd_hbm_bytes_per_launch"]) == 2000 * 1024 * 2 + 500 * 1024


def test_mfma_summary_arithmetic(tmp_path):
    w = synth.WORKLOADS[1]
    nnzb = int(synth.block_mask(w, 0).sum())
    useful = 2.0 * w.M * w.b * w.b * nnzb
    fwd = PREFIX + "k_panel_gemm<32, 2, 4, 4, 4, 2, 1, false, false>(unsigned short const*)"
    rows = []
    for d in (1, 2):   # two dispatches, each counter split over two dimension rows
        for half in (0, 1):
            rows += [{"Dispatch_Id": d, "Kernel_Name": fwd, "Counter_Name": "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                      "Counter_Value": useful / 512 / 2},
                     {"Dispatch_Id": d, "Kernel_Name": fwd, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES",
                      "Counter_Value": 0.25 * 1000 * bench.SIMDS / 2},
                     {"Dispatch_Id": d, "Kernel_Name": fwd, "Counter_Name": "GRBM_GUI_ACTIVE",
                      "Counter_Value": 1000 * bench.XCCS / 2}]
    _write(str(tmp_path / "m" / "run_counter_collection.csv"), rows)
    out = str(tmp_path / "mfma.txt")
    bench.summarize_mfma(str(tmp_path / "m"), w.name, out_path=out)
    line = [ln for ln in open(out) if ln.startswith("| `k_panel_gemm")][0]
    cells = [c.strip() for c in line.strip().strip("|").split("|")]
    assert cells[1] == "fwd" and cells[2] == "2"
    assert abs(float(cells[3]) - useful) <= 1e-6 * useful
    assert cells[4] == "1.000" and cells[5] == "25.0%"


def test_rotation_counts_distinct_bytes():
    """Each buffer set holds every tensor of the step once (X, V, dY, Y, dX, dV); the cold rotation
    must hold at least 512 MiB of distinct buffers, with no set counted twice."""
    for k, w in synth.WORKLOADS.items():
        nnzb = int(synth.block_mask(w, 0).sum())
        one = bench.set_bytes(w, nnzb)
        b2 = 2 * nnzb * w.b * w.b
        expect = 2 * w.M * w.K + b2 + 2 * w.M * w.N + (2 * w.N if w.bias else 0)
        if "dx" in w.ops:
            expect += 2 * w.M * w.N + 2 * w.M * w.K + b2
        assert one == expect, k
        n = bench.rotation_sets(w, nnzb, warm=False)
        assert n * one >= bench.ROTATE_BYTES and (n - 1) * one < bench.ROTATE_BYTES
        assert bench.rotation_sets(w, nnzb, warm=True) == 1
    # BERT-base FFN-up: 65.3 MB per set -> 9 sets (8 would hold 522 MB < 512 MiB = 536.9 MB)
    w2 = synth.WORKLOADS[2]
    assert bench.rotation_sets(w2, int(synth.block_mask(w2, 0).sum()), False) == 9
    # the Zipf layer's one set is already ~1 GB
    w5 = synth.WORKLOADS[5]
    assert bench.rotation_sets(w5, int(synth.block_mask(w5, 0).sum()), False) == 1


def test_headline_is_the_largest_workload():
    w = synth.WORKLOADS[bench.HEADLINE_WORKLOAD]
    flops = {k: 2 * x.M * x.b * x.b * int(synth.block_mask(x, 0).sum()) * len(x.ops)
             for k, x in synth.WORKLOADS.items()}
    assert w.name == "zipf_16384x4096x11008_b32_d0.30"
    assert flops[bench.HEADLINE_WORKLOAD] == max(flops.values())
