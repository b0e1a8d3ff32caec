"""The rocprofv3 harness's digest (CPU only): synthetic CSV files in the
layout rocprofv3 writes (kernel trace, counter collection), the per-kernel
figures derived from them."""
import csv
import os

import pytest

from sparse_expert_ffn_amd import rocprof_report as rr

UP = "void moe::upgate_kernel<unsigned short, 256, 128, false>(moe::ForwardParams)"
DOWN = "void moe::down_kernel<unsigned short, 256, 128, false>(moe::ForwardParams)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _trace(d, rows):
    _write(os.path.join(d, "host", "123_kernel_trace.csv"),
           ["Kind", "Agent_Id", "Queue_Id", "Kernel_Id", "Kernel_Name", "Correlation_Id",
            "Start_Timestamp", "End_Timestamp"],
           [["KERNEL_DISPATCH", 1, 1, 7, n, i, t0, t1] for i, (n, t0, t1) in enumerate(rows)])


def _counters(d, rows):
    """rows: (dispatch, kernel, counter, value, start, end)"""
    _write(os.path.join(d, "host", "123_counter_collection.csv"),
           ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Kernel_Name", "Counter_Name",
            "Counter_Value", "Start_Timestamp", "End_Timestamp"],
           [[i, disp, 1, n, c, v, t0, t1] for i, (disp, n, c, v, t0, t1) in enumerate(rows)])


def test_short_name():
    assert rr.short_name(UP) == "upgate_kernel<unsigned short, 256, 128, false>"
    assert rr.short_name("void moe::f<(anonymous namespace)::X>(int, float)") == \
        "f<(anonymous namespace)::X>"
    assert rr.short_name(COPY) == COPY


def test_digest(tmp_path):
    out = str(tmp_path)
    # two up/gate dispatches of 500 and 540 us, one down of 270 us
    _trace(os.path.join(out, "trace"), [(UP, 0, 500_000), (UP, 1_000_000, 1_540_000),
                                        (DOWN, 2_000_000, 2_270_000)])
    # FETCH_SIZE reported in two rows (dimensions) for one dispatch: summed
    _counters(os.path.join(out, "fetch"), [(1, UP, "FETCH_SIZE", 300_000, 0, 1),
                                           (1, UP, "FETCH_SIZE", 352_000, 0, 1),
                                           (2, UP, "FETCH_SIZE", 652_000, 0, 1)])
    _counters(os.path.join(out, "write"), [(1, UP, "WRITE_SIZE", 128_000, 0, 1)])
    # the copy of 1 GiB read 524288 KiB of FETCH_SIZE (x2 scale), 1048576 KiB of WRITE_SIZE
    _counters(os.path.join(out, "cfetch"), [(1, COPY, "FETCH_SIZE", 524_288, 0, 1)])
    _counters(os.path.join(out, "cwrite"), [(1, COPY, "WRITE_SIZE", 1_048_576, 0, 1)])
    dur = 520_000  # ns
    cyc = 2.0e9 * dur * 1e-9 * rr.XCDS      # 2 GHz, summed over the XCDs
    sq = [(1, UP, "GRBM_GUI_ACTIVE", cyc, 0, dur), (1, UP, "GRBM_COUNT", cyc, 0, dur),
          (1, UP, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cyc / rr.XCDS * rr.SIMDS, 0, dur),
          (1, UP, "SQ_LDS_IDX_ACTIVE", 0.25 * cyc / rr.XCDS * rr.CUS, 0, dur),
          (1, UP, "SQ_LDS_BANK_CONFLICT", 0.0, 0, dur),
          (1, UP, "SQ_WAVE_CYCLES", 1000.0, 0, dur), (1, UP, "SQ_WAIT_INST_ANY", 340.0, 0, dur)]
    _counters(os.path.join(out, "sq"), sq)
    d = rr.digest(out, {"upgate_kernel": {"flops": 533.5e9, "bytes": 1.141e9}})
    assert d["fetch_scale"] == pytest.approx(2.0)
    assert d["write_scale"] == pytest.approx(1.0)
    up = d["kernels"][0]
    assert up["kernel"].startswith("upgate_kernel") and up["calls"] == 2
    assert up["avg_us"] == pytest.approx(520.0)
    assert up["share"] == pytest.approx(1040 / 1310)
    assert up["hbm_read_bytes"] == pytest.approx(652_000 * 1024 * 2.0)
    assert up["hbm_write_bytes"] == pytest.approx(128_000 * 1024)
    assert up["mfma_busy"] == pytest.approx(0.5)
    assert up["lds_active"] == pytest.approx(0.25)
    assert up["wait_issue"] == pytest.approx(0.34)
    assert up["clock_ghz"] == pytest.approx(2.0)
    assert up["tflops"] == pytest.approx(533.5e9 / 520e-6 / 1e12)
    assert up["mfma_frac"] == pytest.approx(up["tflops"] / rr.PEAK_BF16_TFLOPS)
    down = d["kernels"][1]
    assert down["calls"] == 1 and down["hbm_read_bytes"] is None and "tflops" not in down
    md = rr.markdown(d, "t", ["cmd"])
    assert "`upgate_kernel<unsigned short, 256, 128, false>`" in md and "50.0%" in md
    rec = rr.traffic_record(d, "prefill_bal", 256, ["cmd"])
    assert rec["hbm_bytes_per_launch"] == pytest.approx(652_000 * 2048 + 128_000 * 1024)
