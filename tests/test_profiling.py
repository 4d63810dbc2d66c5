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


def test_kernel_labels():
    assert profiling._kernel_label(MANGLED % 0) == "osdn_fused_forward"
    assert profiling._kernel_label(MANGLED % 3) == "osdn_fused_scan"
    assert profiling._kernel_label("osdn::osdn_fused_forward<2>(...)") == "osdn_fused_chunk"
    assert profiling._kernel_label("__amd_rocclr_copyBuffer") is None


def test_means_pick_the_three_largest_copies(tmp_path):
    rows = [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 7.0)]  # a small unrelated copy
    rows += [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 100.0)] * 3
    rows += [(MANGLED % 0, "FETCH_SIZE", 10.0), (MANGLED % 0, "FETCH_SIZE", 14.0),
             (MANGLED % 1, "WRITE_SIZE", 99.0)]
    m = profiling._means(_write(tmp_path, rows), "FETCH_SIZE")
    assert m["copy"] == (100.0, 3)
    assert m["osdn_fused_forward"] == (12.0, 2)
    assert "osdn_fused_deltanet" not in m


def test_summary_table(tmp_path):
    p = tmp_path / "k.csv"
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"])
        w.writerow([MANGLED % 0, 4, 2000000, 500000, 100.0])
    text = profiling.summary(str(p), "cmd")
    assert text.startswith("command: cmd")
    assert "500.000" in text and " 4 " in text
