"""The rocprofv3 summary arithmetic (mixture_experts_ffn_02_amd/profiling.py)
on synthetic counter files: the copy calibration picks the copy kernel only,
read and write bytes are scaled separately, --large keeps the data-moving
dispatches of a kernel launched both ways, and the matrix-core summary
normalises busy cycles by the SIMD count and the per-XCD cycle count."""
import csv
import os

import pytest

from mixture_experts_ffn_02_amd import profiling

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size", "Kernel_Id",
          "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count",
          "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, float, " \
       "at::native::binary_internal::MulFunctor<float> > >"
FILL = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float> >"


def write_counters(path, rows):
    """rows: (dispatch id, kernel, counter, value, duration ns)."""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        for did, kern, ctr, val, dur in rows:
            r = {k: 0 for k in FIELDS}
            r.update(Dispatch_Id=did, Kernel_Name=kern, Counter_Name=ctr, Counter_Value=val, Start_Timestamp=1000,
                     End_Timestamp=1000 + dur)
            w.writerow(r)


def summary(text):
    out = {}
    for line in text.splitlines():
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def test_traffic_scales_reads_and_writes_by_the_copy(tmp_path, capsys):
    copy_bytes = 256 << 20
    # the copy reads 256 MiB that FETCH_SIZE reports as half (128-byte requests
    # counted as 64), writes 256 MiB exactly; a fill kernel in the same run
    # reads nothing and must not enter the calibration
    fetch = [(1, FILL, "FETCH_SIZE", 0.0, 10), (2, COPY, "FETCH_SIZE", copy_bytes / 2048, 10),
             (3, "k_gemm8<true, true, false>", "FETCH_SIZE", 3000.0, 10),
             (4, "k_gemm8<true, true, false>", "FETCH_SIZE", 5000.0, 10)]
    write = [(1, FILL, "WRITE_SIZE", copy_bytes / 1024, 10), (2, COPY, "WRITE_SIZE", copy_bytes / 1024, 10),
             (3, "k_gemm8<true, true, false>", "WRITE_SIZE", 100.0, 10),
             (4, "k_gemm8<true, true, false>", "WRITE_SIZE", 300.0, 10)]
    rdreq = [(2, COPY, "TCC_EA0_RDREQ_128B_sum", copy_bytes / 128, 10), (2, COPY, "TCC_EA0_RDREQ_64B_sum", 0, 10),
             (2, COPY, "TCC_EA0_RDREQ_32B_sum", 0, 10),
             (3, "k_gemm8<true, true, false>", "TCC_EA0_RDREQ_128B_sum", 8000 * 1024 / 128, 10),
             (3, "k_gemm8<true, true, false>", "TCC_EA0_RDREQ_64B_sum", 0, 10),
             (3, "k_gemm8<true, true, false>", "TCC_EA0_RDREQ_32B_sum", 0, 10)]
    write_counters(tmp_path / "f", fetch)
    write_counters(tmp_path / "w", write)
    write_counters(tmp_path / "r", rdreq)
    profiling.main(["traffic", "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"), "--rdreq",
                    str(tmp_path / "r"), "--kernel", "k_gemm8<true, true", "--copy-bytes", str(copy_bytes),
                    "--algorithmic", str(4000 * 1024), "--cmd", "x"])
    s = summary(capsys.readouterr().out)
    assert float(s["fetch_scale"]) == pytest.approx(2.0)
    assert float(s["write_scale"]) == pytest.approx(1.0)
    # mean over the two dispatches: reads (3000 + 5000) / 2 KiB x 2, writes (100 + 300) / 2 KiB
    assert float(s["read_bytes_per_launch"]) == pytest.approx(8000 * 1024)
    assert float(s["write_bytes_per_launch"]) == pytest.approx(200 * 1024)
    assert float(s["hbm_bytes_per_launch"]) == pytest.approx(8200 * 1024)
    assert float(s["traffic_over_algorithmic"]) == pytest.approx(8200 / 4000, rel=1e-3)
    assert float(s["rdreq_over_scaled_fetch"]) == pytest.approx(1.0, rel=1e-3)


def test_traffic_large_keeps_the_data_moving_dispatches(tmp_path, capsys):
    copy_bytes = 1 << 20
    fetch = [(1, COPY, "FETCH_SIZE", 512.0, 10), (2, "k_scatter(int)", "FETCH_SIZE", 1.0, 10),
             (3, "k_scatter(int)", "FETCH_SIZE", 900.0, 10), (4, "k_scatter(int)", "FETCH_SIZE", 1100.0, 10)]
    write = [(1, COPY, "WRITE_SIZE", 1024.0, 10), (2, "k_scatter(int)", "WRITE_SIZE", 2.0, 10),
             (3, "k_scatter(int)", "WRITE_SIZE", 7000.0, 10), (4, "k_scatter(int)", "WRITE_SIZE", 9000.0, 10)]
    write_counters(tmp_path / "f", fetch)
    write_counters(tmp_path / "w", write)
    profiling.main(["traffic", "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"), "--kernel",
                    "k_scatter", "--large", "--copy-bytes", str(copy_bytes), "--cmd", "x"])
    s = summary(capsys.readouterr().out)
    assert s["dispatches"] == "2"
    assert float(s["read_bytes_per_launch"]) == pytest.approx(1000 * 2 * 1024)
    assert float(s["write_bytes_per_launch"]) == pytest.approx(8000 * 1024)


def test_mfma_busy_and_clock(tmp_path, capsys):
    # 1 ms at 1.5 GHz: 1.5e6 cycles per XCD, 8 XCDs summed; 1024 SIMDs busy 75%
    cyc = 1.5e6
    rows = [(1, "k_gemm8<true, true, false>", "GRBM_GUI_ACTIVE", 8 * cyc, 1_000_000),
            (1, "k_gemm8<true, true, false>", "SQ_VALU_MFMA_BUSY_CYCLES", 0.75 * 1024 * cyc, 1_000_000),
            (1, "k_gemm8<true, true, false>", "SQ_INSTS_VALU_MFMA_MOPS_BF16", 2e12 / 512, 1_000_000)]
    write_counters(tmp_path / "m", rows)
    profiling.main(["mfma", str(tmp_path / "m"), "--kernel", "k_gemm8", "--cmd", "x"])
    line = [l for l in capsys.readouterr().out.splitlines() if "k_gemm8" in l and not l.startswith("#")][0].split()
    launches, busy, ghz, pf, gflop, us = line[:6]
    assert int(launches) == 1
    assert float(busy) == pytest.approx(0.75, abs=1e-3)
    assert float(ghz) == pytest.approx(1.5, abs=1e-2)
    assert float(pf) == pytest.approx(2.5 * 1.5 / 2.4, abs=1e-2)
    assert float(gflop) == pytest.approx(2000.0, rel=1e-3)
    assert float(us) == pytest.approx(1000.0)


def test_bench_work_and_roofline_choice():
    """bench.py's algorithmic work: the DeepSeek-style layer's routed gate/up
    (the shared expert runs on its own) is 4 T k d d_ff flops over the x rows,
    every expert's gate and up weights and H; a batch that touches few experts
    counts only their weights, and its gate/up launch, below the ridge of the
    two peaks, is reported against HBM."""
    import bench
    from mixture_experts_ffn_02_amd.inputs import CONFIGS

    cfg = CONFIGS["deepseek_fine"]
    T, d, k, f, E = cfg.T, cfg.d_model, cfg.top_k, cfg.d_ff, cfg.n_experts
    w = bench.phase_bytes_and_flops(cfg)
    assert w["gateup"]["flops"] == 4.0 * T * k * d * f
    assert w["gateup"]["bytes"] == T * k * d * 2 + E * 2 * f * d * 2 + T * k * f * 2 == 24696061952
    r = bench.gateup_roofline(cfg, w, 28.0, None)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(4.0 * T * k * d * f / 28e-3 / 1e12, rel=1e-3)

    one = cfg.with_tokens(1)
    w1 = bench.phase_bytes_and_flops(one, used=8)
    assert "shared_gateup" not in w1  # the shared expert is one more group of the routed launches
    weights = (8 * 2 * f * d + 2 * f * d) * 2
    assert w1["gateup"]["bytes"] == (k + 1) * d * 2 + weights + (k + 1) * f * 2
    r1 = bench.gateup_roofline(one, w1, 0.1, None)
    assert r1["bound"] == "hbm" and r1["unit"] == "GB/s"
    assert r1["achieved"] == pytest.approx(w1["gateup"]["bytes"] / 0.1e-3 / 1e9, rel=1e-3)
    assert bench.gemm_row_tile((k + 1) * 1, E + 1, f, d) == 64


def test_bench_row_tile_follows_the_library():
    """bench.py names the gate/up kernel and its tile from a Python copy of the
    library's forward row-tile rule; the copy gives the library's own answer
    (its exported host function, with the 256 CUs it assumes when no device
    is visible) on layers from one row to the DeepSeek-style batch, one group
    to 257, and the widths and K of the workload layers."""
    import ctypes

    import bench
    from mixture_experts_ffn_02_amd import _native as N

    lib = N.load()
    cu = getattr(lib, "_ZN3moe8cu_countEv")
    cu.restype = ctypes.c_int
    if cu() != 256:
        pytest.skip("a device with another CU count is visible")
    rule = getattr(lib, "_ZN3moe11gemm_bm_fwdEillii")
    rule.restype = ctypes.c_int
    rule.argtypes = [ctypes.c_int, ctypes.c_long, ctypes.c_long, ctypes.c_int, ctypes.c_int]
    n_checked = 0
    for rows in (1, 3, 24, 100, 1000, 4096, 16384, 36864, 131072, 147456, 524288):
        for groups in (1, 16, 64, 65, 128, 129, 256, 257):
            for n in (64, 192, 256, 768, 1024, 2048, 4352):
                for d_in in (64, 512, 2048, 4096, 5120, 7168):
                    assert bench.gemm_row_tile(rows, groups, n, d_in) == rule(1, rows, groups, n, d_in), \
                        (rows, groups, n, d_in)
                    n_checked += 1
    assert n_checked == 11 * 8 * 7 * 6
