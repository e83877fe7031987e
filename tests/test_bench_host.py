"""Host logic of bench.py (no GPU): the rocprofv3 counter parsing and its
calibration, the matrix-core busy fraction, the XCD fetch model and the
source digest that ties stored counters to a build."""
import csv
import os
import shutil
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
DOM = "void qll::gemm_pipe_kernel<1, 128, 128, 4, 4, 128, 4, false, false, 1>(qll::GemmArgs)"
CAL = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float>>(int)"


def write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": k, "Counter_Name": c,
                        "Counter_Value": v})


def test_counter_per_dispatch_groups_by_kernel(tmp_path):
    p = tmp_path / "c.csv"
    write_counters(p, [(DOM, "FETCH_SIZE", 10.0), (CAL, "FETCH_SIZE", 3.0),
                       (DOM, "FETCH_SIZE", 30.0), (DOM, "WRITE_SIZE", 7.0)])
    d = bench.counter_per_dispatch(str(p), "FETCH_SIZE")
    assert d == {DOM: [10.0, 30.0], CAL: [3.0]}


def test_hbm_traffic_scales_by_the_calibration_copy(tmp_path):
    # the copy reads and writes CALIB_BYTES; its counters read half of that
    # (factor 2), so the dominant kernel's mean KiB count doubles
    cal_kib = bench.CALIB_BYTES / 1024.0 / 2
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    write_counters(fetch, [(CAL, "FETCH_SIZE", 16.0), (CAL, "FETCH_SIZE", cal_kib),
                           (DOM, "FETCH_SIZE", 1000.0), (DOM, "FETCH_SIZE", 3000.0)])
    write_counters(write, [(CAL, "WRITE_SIZE", cal_kib), (DOM, "WRITE_SIZE", 500.0)])
    tr = bench.hbm_traffic(str(fetch), str(write), "void qll::gemm_pipe_kernel<1, 128")
    assert tr["FETCH_SIZE_factor"] == pytest.approx(2.0)
    assert tr["FETCH_SIZE"] == pytest.approx(2000.0 * 1024 * 2)
    assert tr["WRITE_SIZE"] == pytest.approx(500.0 * 1024 * 2)
    assert tr["bytes_per_launch"] == pytest.approx((2000.0 + 500.0) * 1024 * 2)
    # no calibration copy in the run: no figure rather than an unscaled one
    write_counters(write, [(DOM, "WRITE_SIZE", 500.0)])
    assert bench.hbm_traffic(str(fetch), str(write), "void qll::gemm_pipe_kernel") is None


def test_mfma_busy_fraction(tmp_path):
    p = tmp_path / "m.csv"
    cus = 256
    gui = 8 * 1000.0                      # summed over the 8 XCDs: 1000 cycles each
    busy = 0.25 * 1000.0 * 4 * cus        # a quarter of the SIMD cycles
    write_counters(p, [(DOM, "SQ_VALU_MFMA_BUSY_CYCLES", busy), (DOM, "GRBM_GUI_ACTIVE", gui)])
    mb = bench.mfma_busy(str(p), "void qll::gemm_pipe_kernel", cus)
    assert mb["mfma_busy_frac"] == pytest.approx(0.25)
    assert mb["dispatches"] == 1


def test_mfma_counters_calibration(tmp_path):
    # busy cycles = instructions x 32, MOPS x 512 = the algorithmic flops,
    # clock = GRBM_GUI_ACTIVE / 8 XCDs / the dispatch's duration
    p = tmp_path / "m.csv"
    def write(end_ns, gui):
        rows = [(DOM, "SQ_VALU_MFMA_BUSY_CYCLES", 32.0 * 4096), (DOM, "SQ_INSTS_MFMA", 4096.0),
                (DOM, "SQ_INSTS_VALU_MFMA_MOPS_F8", 1e6 / 512), (DOM, "GRBM_GUI_ACTIVE", gui)]
        with open(p, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=FIELDS + ["Start_Timestamp", "End_Timestamp"])
            w.writeheader()
            for k, c, v in rows:
                w.writerow({"Dispatch_Id": 1, "Kernel_Name": k, "Counter_Name": c,
                            "Counter_Value": v, "Start_Timestamp": 1000, "End_Timestamp": end_ns})
    write(201000, 8 * 400000.0)  # a 200 us dispatch at 2 GHz
    mb = bench.mfma_busy(str(p), "void qll::gemm_pipe_kernel", 256, flops_per_launch=1e6)
    assert mb["busy_cycles_per_mfma"] == 32.0
    assert mb["mops_f8_flops"] == 1000000
    assert mb["mops_over_algorithmic"] == pytest.approx(1.0)
    assert mb["dispatch_us"] == pytest.approx(200.0)
    assert mb["clock_ghz"] == pytest.approx(2.0)
    # a short dispatch: the counter's wider window would inflate the clock
    write(11000, 8 * 20000.0)
    mb = bench.mfma_busy(str(p), "void qll::gemm_pipe_kernel", 256, flops_per_launch=1e6)
    assert mb["dispatch_us"] == pytest.approx(10.0) and "clock_ghz" not in mb


def write_trace(path, kernels):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 0
        for k, dur in kernels:
            w.writerow({"Kernel_Name": k, "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + 100


def test_trace_timed_durations_picks_the_timed_replays(tmp_path):
    # 3 step dispatches, then problem 0 (copies 2, replays 3): 2 untimed, 6
    # timed, 8 warm; then problem 4 (copies 1, replays 3): 1, 3, 4; another
    # kernel interleaved is ignored
    other = "void qll::splitk_reduce_kernel<1>(qll::GemmArgs)"
    seq = [(DOM, 1)] * 3 + [(DOM, 2)] * 2 + [(DOM, 1000)] * 6 + [(other, 5)] + [(DOM, 3)] * 8
    seq += [(DOM, 4)] + [(DOM, 2000)] * 3 + [(DOM, 7)] * 4
    p = tmp_path / "t.csv"
    write_trace(p, seq)
    td = bench.trace_timed_durations(str(p), DOM, 3, [(0, 2, 3), (4, 1, 3)])
    assert td == {0: [1.0] * 6, 4: [2.0] * 3}
    # a count that does not match the plan: no figure
    assert bench.trace_timed_durations(str(p), DOM, 4, [(0, 2, 3), (4, 1, 3)]) is None


def test_xcd_fill_bytes_bounds():
    # one tile per XCD: every XCD fetches exactly its own rows (no sharing)
    M, N, K, bp, bq = 256, 512, 1024, 128, 128
    assert bench.xcd_fill_bytes(M, N, K, bp, bq) == 8 * (bp + bq) * K
    # many tiles: between the algorithmic bytes (each row once on the whole
    # chip) and every tile reading its own rows
    M, N, K = 2048, 2048, 6144
    got = bench.xcd_fill_bytes(M, N, K, 128, 128)
    tiles = (M // 128) * (N // 128)
    assert (M + N) * K <= got <= tiles * (128 + 128) * K
    # ragged edges count only the rows that exist
    assert bench.xcd_fill_bytes(100, 60, 256, 128, 128) == (100 + 60) * 256


def test_source_digest_follows_the_sources(tmp_path, monkeypatch):
    d0 = bench.source_digest()
    assert len(d0) == 16 and int(d0, 16) >= 0
    assert bench.source_digest() == d0
    root = tmp_path / "repo"
    shutil.copytree(os.path.join(bench.ROOT, "quantized_linear_layer_scaled_amd", "csrc"),
                    root / "quantized_linear_layer_scaled_amd" / "csrc")
    shutil.copytree(os.path.join(bench.ROOT, "include"), root / "include")
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.source_digest() == d0
    with open(root / "quantized_linear_layer_scaled_amd" / "csrc" / "api.cpp", "a") as f:
        f.write("\n")
    assert bench.source_digest() != d0


def test_kernel_symbol_matches_the_demangled_pipe_kernels():
    # the names rocprofv3 prints for the pipelined kernels carry every
    # template argument, the K-group count included; bench.py must build
    # the same string to find the dominant kernel in a trace
    import quantized_linear_layer_scaled_amd as qll
    qll.load_library()
    assert bench.kernel_symbol(qll, "fp8", "p128x128_w4x4_k128_s3") == (
        "void qll::gemm_pipe_kernel<1, 128, 128, 4, 4, 128, 3, false, false, 1>(qll::GemmArgs)")
    assert bench.kernel_symbol(qll, "int8", "p64x64_w2x2_k128_s4_g2") == (
        "void qll::gemm_pipe_kernel<0, 64, 64, 2, 2, 128, 4, false, false, 2>(qll::GemmArgs)")
    assert bench.kernel_symbol(qll, "fp8_grouped", "p256x256_w2x4_k128_s2") == (
        "void qll::gemm_pipe_kernel<1, 256, 256, 2, 4, 128, 2, false, true, 1>(qll::GemmArgs)")
    assert bench.kernel_symbol(qll, "fp8", "p128x128_w2x4_k128_r2") == (
        "void qll::gemm_pipe_rc_kernel<1, 128, 128, 2, 4, 128, 2, false>(qll::GemmArgs)")
