"""The rocprofv3 summary helper that writes the counter record bench.py
reads (CPU only: synthetic CSV files in rocprofv3's column layout)."""
import csv
import json

from bit_companded_adam_amd import rocprof_summary as S

COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
        "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
        "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
        "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write(d, rows):
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, COLS)
        w.writeheader()
        for r in rows:
            w.writerow({c: r.get(c, 0) for c in COLS})


def _row(disp, kernel, counter, value, t0=0, t1=10_000_000):
    return {"Dispatch_Id": disp, "Kernel_Name": kernel, "Counter_Name": counter,
            "Counter_Value": value, "Start_Timestamp": t0, "End_Timestamp": t1}


def test_short_name():
    n = "void flashopt::(anonymous namespace)::adamw_step_kernel<24, 1>(flashopt::StepScalars const*, int)"
    assert S.short_name(n) == "flashopt::adamw_step_kernel<24, 1>"


def test_counter_record(tmp_path):
    k = "void flashopt::(anonymous namespace)::adamw_step_kernel<24, 1>(int)"
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int)"
    cal = 2 << 30
    # the copy's FETCH_SIZE reads half its bytes, WRITE_SIZE all (KiB)
    _write(tmp_path / "cf", [_row(1, neg, "FETCH_SIZE", cal / 2 / 1024)])
    _write(tmp_path / "cw", [_row(1, neg, "WRITE_SIZE", cal / 1024)])
    n = 1 << 20
    # two step dispatches, 10 ms each; the second is the steady step
    _write(tmp_path / "f", [_row(7, k, "FETCH_SIZE", 1.0), _row(8, k, "FETCH_SIZE", 7.125 * n / 2 / 1024)])
    _write(tmp_path / "w", [
        _row(7, k, "WRITE_SIZE", 1.0), _row(7, k, "SQ_INSTS_VALU", 10.0),
        _row(8, k, "WRITE_SIZE", 5.125 * n / 1024), _row(8, k, "SQ_INSTS_VALU", 65.0 * n / 64),
        _row(8, k, "GRBM_GUI_ACTIVE", 8 * 16_000_000)])
    out = tmp_path / "rec.json"
    S.main(["counters", "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"),
            "--cal-fetch", str(tmp_path / "cf"), "--cal-write", str(tmp_path / "cw"),
            "--params", str(n), "--alg-read", "7.125", "--alg-write", "5.125", "--json", str(out)])
    rec = json.load(open(out))
    assert abs(rec["fetch_factor"] - 2.0) < 1e-12 and rec["write_factor"] == 1.0
    assert abs(rec["hbm_bytes_per_launch"] - 12.25 * n) < 1e-6 * n
    assert abs(rec["valu_per_element_lane"] - 65.0) < 1e-9
    assert abs(rec["sclk_mhz_during_step"] - 1600.0) < 1e-6      # 16e6 cycles per XCD in 10 ms
    assert rec["valu_first_step"] == 10.0
