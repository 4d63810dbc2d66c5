"""Host-side logic of the profiling helpers (no GPU): kernel labels, counter
means with the copy calibration, and the kernel-time table."""
import csv
import os

from delta_rule_recurrent_precond_amd import profiling

HEADER = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
MANGLED = "_ZN4osdn12_GLOBAL__N_118osdn_fused_forwardILi%dEEEvPKDF16b"


def _write(tmp_path, rows):
    d = tmp_path / "pmc"
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HEADER)
        for i, (name, counter, value) in enumerate(rows):
            w.writerow([i + 1, i + 1, name, counter, value])
    return str(d)


def test_library_kernels():
    assert profiling._is_library_kernel(MANGLED % 0)
    assert profiling._is_library_kernel("osdn::(anonymous namespace)::chunk_state(...)")
    assert not profiling._is_library_kernel("__amd_rocclr_copyBuffer")
    assert not profiling._is_library_kernel("void at::native::vectorized_elementwise_kernel")


def test_totals_sum_library_kernels_and_pick_the_three_largest_copies(tmp_path):
    rows = [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 7.0)]  # a small unrelated copy
    rows += [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 100.0)] * 3
    rows += [(MANGLED % 0, "FETCH_SIZE", 10.0), (MANGLED % 0, "FETCH_SIZE", 14.0),
             ("osdn::walk(...)", "FETCH_SIZE", 5.0), (MANGLED % 1, "WRITE_SIZE", 99.0)]
    copy_mean, lib = profiling._totals(_write(tmp_path, rows), "FETCH_SIZE")
    assert copy_mean == 100.0
    assert lib[MANGLED % 0] == (24.0, 2)
    assert lib["osdn::walk(...)"] == (5.0, 1)
    assert MANGLED % 1 not in lib


def test_record_divides_by_calls(tmp_path, monkeypatch):
    rows_f = [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 1024.0)] * 3
    rows_f += [("osdn::walk(...)", "FETCH_SIZE", 64.0)] * 2
    rows_w = [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 2048.0)] * 3
    rows_w += [("osdn::walk(...)", "WRITE_SIZE", 8.0)] * 2
    df = tmp_path / "f"
    dw = tmp_path / "w"
    df.mkdir()
    dw.mkdir()
    for d, rows in ((df, rows_f), (dw, rows_w)):
        with open(d / "run_counter_collection.csv", "w", newline="") as f:
            wr = csv.writer(f)
            wr.writerow(HEADER)
            for i, (name, counter, value) in enumerate(rows):
                wr.writerow([i + 1, i + 1, name, counter, value])
    monkeypatch.setattr(profiling, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    profiling.record(str(df), str(dw), "wl", "scan_split", 2, "cf", "cw")
    import json
    rec = json.load(open(tmp_path / "profiles" / "traffic.json"))["osdn_precond_scan_split|wl"]
    # 2 dispatches x 64 units x (2^30 / 1024) bytes per unit, over 2 calls
    assert rec["fetch_bytes"] == 64 * (1 << 30) / 1024
    assert rec["write_bytes"] == 8 * (1 << 30) / 2048


def test_summary_table(tmp_path):
    p = tmp_path / "k.csv"
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"])
        w.writerow([MANGLED % 0, 4, 2000000, 500000, 100.0])
    text = profiling.summary(str(p), "cmd")
    assert text.startswith("command: cmd")
    assert "500.000" in text and " 4 " in text


def test_record_mfma_counts_512_flop_units_per_call(tmp_path, monkeypatch):
    rows = []
    for disp, (name, f16, f32, busy, cu) in enumerate([("osdn::chunk_state(...)", 10.0, 0.0, 30.0, 60.0),
                                                       ("osdn::chunk_state(...)", 14.0, 0.0, 30.0, 60.0),
                                                       ("osdn::walk_prep(...)", 2.0, 4.0, 5.0, 50.0),
                                                       ("__amd_rocclr_copyBuffer", 99.0, 99.0, 9.0, 9.0)]):
        for c, v in zip(profiling.MFMA_COUNTERS, (f16, f32, busy, cu)):
            rows.append((disp, name, c, v))
    d = tmp_path / "m"
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(HEADER)
        for i, (disp, name, counter, value) in enumerate(rows):
            wr.writerow([i + 1, disp + 1, name, counter, value])
    monkeypatch.setattr(profiling, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    profiling.record_mfma(str(d), "wl", "forward_split", 2, "cmd")
    import json
    rec = json.load(open(tmp_path / "profiles" / "mfma.json"))["osdn_forward_split|wl"]
    assert rec["f16_flops_per_call"] == (10 + 14 + 2) * 512 / 2
    assert rec["f32_flops_per_call"] == 4 * 512 / 2
    text = open(tmp_path / "profiles" / "mfma_forward_split_wl.txt").read()
    assert "0.500" in text and "0.100" in text  # busy shares 60/120 and 5/50
