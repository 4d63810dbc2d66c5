"""Host-side arithmetic of bench.py (no GPU): the algorithmic bytes and flops
the roofline fields divide by, and the rule that stored counter figures only
count for the kernel sources they were taken from."""
import json

import bench
from delta_rule_recurrent_precond_amd import workloads as W


def test_algorithmic_bytes_of_the_metric_workload():
    w = W.METRIC_WORKLOAD
    th, heads = w.B * w.H * w.T, w.B * w.H
    # q, k, v read and o written in bf16 (128 elements each), beta and r in fp32;
    # per head S_final (128 x 128 fp32) and d_final (128 fp32)
    per = 4 * 128 * 2 + 4 + 4
    assert bench.algorithmic_bytes(w, "fused") == th * per + heads * (128 * 128 * 4 + 128 * 4)
    assert bench.algorithmic_bytes(w, "fused") == 274_759_680
    # the chunk pass also reads kt and handles no r or d
    assert bench.algorithmic_bytes(w, "chunk") == th * (5 * 128 * 2 + 4) + heads * 128 * 128 * 4
    # the walk reads k, beta, r and writes kt, plus d_final
    assert bench.algorithmic_bytes(w, "scan") == th * (2 * 128 * 2 + 8) + heads * 128 * 4


def test_algorithmic_flops_of_the_metric_workload():
    w = W.METRIC_WORKLOAD
    C, dk, dv = w.chunk, w.dk, w.dv
    # chunk pass: three state contractions (K S^T, Q S^T, S update) at 2 dk dv
    # each, the gram, W and the scores at 2 C dk each, U and scores X at 2 C dv
    # each, the inverse C^2 / 3; the walk about 8 dk
    per = 3 * 2 * dk * dv + 3 * 2 * C * dk + 2 * 2 * C * dv + C * C / 3 + 8 * dk
    assert bench.algorithmic_flops(w) == int(w.B * w.H * w.T * per)
    assert abs(bench.algorithmic_flops(w) / 1e9 - 47.87) < 0.01


def test_stored_figures_only_count_for_their_kernel_sources(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    rec = {"osdn_forward_split|1.3b-apf": {"sources": "current", "bytes_per_launch": 9.0e8,
                                           "f16_flops_per_call": 4.0e10, "f32_flops_per_call": 1.0}}
    json.dump(rec, open(tmp_path / "profiles" / "traffic.json", "w"))
    json.dump(rec, open(tmp_path / "profiles" / "mfma.json", "w"))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sources_hash", lambda: "current")
    assert bench.stored_traffic("osdn_forward_split", "1.3b-apf") == 9.0e8
    assert bench.stored_mfma("osdn_forward_split", "1.3b-apf") == {"f16_flops": 4.0e10,
                                                                   "f32_flops": 1.0}
    assert bench.stored_traffic("osdn_forward_split", "other") is None
    monkeypatch.setattr(bench, "kernel_sources_hash", lambda: "changed")
    assert bench.stored_traffic("osdn_forward_split", "1.3b-apf") is None
    assert bench.stored_mfma("osdn_forward_split", "1.3b-apf") is None
