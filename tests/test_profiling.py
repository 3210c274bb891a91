"""Host-side checks of the rocprofv3 summariser used for profiles/."""
import csv
import json

from adaptive_sparse_attention_amd import profiling


def _counter_csv(path, counter, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for i, (k, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})


def test_short_name():
    assert profiling.short_name("void ea::fwd_out_kernel<ea::BF16, 64, 1, 2>(ea::FwdArgs)") == \
        "fwd_out_kernel<BF16, 64, 1, 2>"
    assert profiling.base_name("void ea::fwd_out_kernel<ea::BF16, 64, 1, 2>(ea::FwdArgs)") == "fwd_out_kernel"


def test_traffic_calibration(tmp_path):
    k = "void ea::bwd_rows_kernel<ea::BF16, 64, 1, 2>(ea::BwdArgs)"
    cp = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int, float)"
    # the copy moves 1 MiB each way; the fetch counter reads half of it
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [(k, 100.0), (k, 300.0), (cp, 512.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [(k, 50.0), (k, 50.0), (cp, 1024.0)])
    out = tmp_path / "t.txt"
    js = tmp_path / "t.json"
    rc = profiling.main(["traffic", "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
                         "--copy-bytes", str(1 << 20), "--command", "c", "--out", str(out), "--json", str(js)])
    assert rc == 0
    rec = json.loads(js.read_text())
    e = rec["bwd_rows_kernel"]
    assert e["fetch_bytes"] == 200.0 * 1024 * 2
    assert e["write_bytes"] == 50.0 * 1024
    assert e["traffic_bytes_per_launch"] == e["fetch_bytes"] + e["write_bytes"]
    assert e["source_sha"] == profiling.kernel_source_sha()
    assert rec["_calibration"]["fetch_factor"] == 2.0


def test_stats_table(tmp_path):
    p = tmp_path / "s.csv"
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow(["void ea::a_kernel<ea::BF16>(ea::FwdArgs)", 2, 2000000, 1000000, 25.0, 1, 1, 0])
        w.writerow(["void ea::b_kernel<ea::BF16>(ea::FwdArgs)", 2, 6000000, 3000000, 75.0, 1, 1, 0])
    rows = profiling.stats_table(str(p))
    assert rows[0][0] == "b_kernel<BF16>" and abs(rows[0][2] - 3.0) < 1e-12


def test_counter_metrics(tmp_path):
    k = "void ea::fwd_init_kernel<ea::BF16, 64>(ea::FwdArgs)"
    rows = [("GRBM_GUI_ACTIVE", 1000.0), ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 2.4 * 250.0), ("SQ_INSTS_MFMA", 100.0),
            ("SQ_INSTS_VALU", 400.0), ("SQ_INSTS_SALU", 50.0), ("SQ_WAIT_ANY", 30.0), ("SQ_WAVE_CYCLES", 120.0),
            ("SQ_INSTS_LDS", 80.0), ("SQ_LDS_BANK_CONFLICT", 20.0), ("SQ_ACTIVE_INST_LDS", 160.0),
            ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 2.0)]
    p = tmp_path / "c.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, v in rows:   # a dispatch of 1000 ns
            w.writerow({"Dispatch_Id": 0, "Kernel_Name": k, "Counter_Name": name, "Counter_Value": v,
                        "Start_Timestamp": 5000, "End_Timestamp": 6000})
    d = profiling.derived(profiling.counter_table([str(p)])[k])
    assert d["mfma_util"] == 0.25
    assert d["mfma_flop"] == 1024.0
    assert d["valu_per_mfma"] == 3.0 and d["salu_per_mfma"] == 0.5
    assert d["wait_frac"] == 0.25
    assert d["lds_conflict_per_inst"] == 0.25 and d["lds_conflict_frac"] == 0.125
    out = tmp_path / "o.txt"
    assert profiling.main(["counters", str(p), "--command", "c", "--out", str(out)]) == 0
    assert "fwd_init_kernel" in out.read_text()
