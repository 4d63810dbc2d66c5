"""Measured HBM traffic and kernel-time summaries for the library's entry points.

HBM bytes per call come from two rocprofv3 counter passes over the same
program (the counter blocks cannot hold FETCH_SIZE and WRITE_SIZE in one pass),
each scaled by what the same counter reads for a device-to-device copy of a
known size run in the same process.  A call may launch several kernels (the
split forward launches four); its bytes are the sum over every library kernel
the program dispatched, divided by the number of calls:

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d D1 -o run -- \\
        python3 -m delta_rule_recurrent_precond_amd.profiling run --entry E
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d D2 -o run -- \\
        python3 -m delta_rule_recurrent_precond_amd.profiling run --entry E
    python3 -m delta_rule_recurrent_precond_amd.profiling record --entry E --fetch D1 --write D2

`record` writes profiles/traffic.json (read by bench.py; an entry only counts
while the kernel sources are unchanged) and a text summary under profiles/.
`mfma` does the same for one pass over MFMA_COUNTERS (matrix-core flops per
call and busy share): profiles/mfma.json and profiles/mfma_<entry>_<workload>.txt.
`summary` turns a rocprofv3 --kernel-trace --stats output (kernel_stats.csv or
the SQLite database) into the text tables kept under profiles/.
"""
from __future__ import annotations

import argparse
import csv
import dataclasses
import glob
import hashlib
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CAL_BYTES = 1 << 30  # calibration copy: 1 GiB read, 1 GiB written
# entry -> the label bench.py looks up in traffic.json
ENTRIES = {
    "forward_split": "osdn_forward_split",
    "forward_fused": "osdn_fused_forward",
    "deltanet_split": "osdn_deltanet_split",
    "scan_split": "osdn_precond_scan_split",
    "chunk_split": "osdn_chunk_fwd_split",
    "forward_gated_split": "osdn_forward_gated_split",
    "forward_raw_split": "osdn_forward_raw_split",
    "forward_kda_split": "osdn_forward_kda_split",
}
# entries that profile another draw of the same workload: the state gate added,
# or q, k unnormalised with beta, r as logits (the kernels transform them)
DRAWS = {"forward_gated_split": {"gated": True}, "forward_raw_split": {"raw": True},
         "forward_kda_split": {"gated": True, "gate_channels": True}}


def kernel_sources_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "delta_rule_recurrent_precond_amd", "csrc", "*"))):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def _is_library_kernel(name: str) -> bool:
    """Kernels of libosdn.so (namespace osdn, mangled or demangled)."""
    return "4osdn" in name or "osdn::" in name


def call(entry: str, dev, w):
    """One call of the entry point on the device inputs."""
    import delta_rule_recurrent_precond_amd as osdn

    if entry == "forward_split":
        osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, eta=dev.eta, chunk=w.chunk)
    elif entry == "forward_fused":
        osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, eta=dev.eta, chunk=w.chunk,
                     workspace=None)
    elif entry == "deltanet_split":
        osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, eta=dev.eta, chunk=w.chunk,
                     precond=False)
    elif entry == "scan_split":
        osdn.precond_scan(dev.k, dev.beta, dev.r, None, dev.eta)
    elif entry == "chunk_split":
        osdn.chunk_fwd(dev.q, dev.k, dev.k, dev.v, dev.beta, chunk=w.chunk)
    elif entry == "forward_gated_split":
        osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, eta=dev.eta, chunk=w.chunk,
                     alpha=dev.alpha)
    elif entry == "forward_kda_split":  # one gate per key dimension
        osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, eta=dev.eta, chunk=w.chunk,
                     alpha=dev.alpha)
    elif entry == "forward_raw_split":
        osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, eta=dev.eta, chunk=w.chunk,
                     norm_qk=True, gate_logits=True)
    else:
        raise SystemExit("unknown entry %s" % entry)


def run(workload: str, launches: int, entry: str) -> None:
    """The program the counter passes profile: a calibration copy, then
    `launches` calls of one entry point on the workload."""
    import torch

    import delta_rule_recurrent_precond_amd as osdn
    from delta_rule_recurrent_precond_amd import workloads as W

    osdn.load()
    a = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    w = dataclasses.replace(W.CONFIGS[workload], **DRAWS.get(entry, {}))
    dev = W.generate(w).to("cuda")
    for _ in range(launches):
        call(entry, dev, w)
    torch.cuda.synchronize()
    print("profiled program done: %s, %s, %d calls" % (workload, entry, launches), flush=True)


def _counter_rows(directory: str):
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % directory)
    rows = []
    for f in files:
        for r in csv.DictReader(open(f)):
            rows.append(r)
    return rows


def _totals(directory: str, counter: str):
    """Mean counter value per dispatch of the calibration copy (the three
    largest copies), and the sum over every library kernel dispatch with the
    per-kernel dispatch counts."""
    per = {}
    for r in _counter_rows(directory):
        if r.get("Counter_Name", "").strip() != counter:
            continue
        name = r.get("Kernel_Name", "")
        key = (name, r.get("Dispatch_Id", r.get("Correlation_Id")))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])  # summed over instances
    copies = sorted(v for (n, _), v in per.items() if "copy" in n.lower())[-3:]
    lib = {}
    for (n, _), v in per.items():
        if _is_library_kernel(n):
            tot, cnt = lib.get(n, (0.0, 0))
            lib[n] = (tot + v, cnt + 1)
    copy_mean = sum(copies) / len(copies) if copies else None
    return copy_mean, lib


def record(fetch_dir: str, write_dir: str, workload: str, entry: str, launches: int,
           cmd_fetch: str, cmd_write: str) -> None:
    copy_f, fetch = _totals(fetch_dir, "FETCH_SIZE")
    copy_w, write = _totals(write_dir, "WRITE_SIZE")
    if not copy_f or not copy_w:
        raise SystemExit("calibration copy not found in the counter output")
    if not fetch or not write:
        raise SystemExit("no library kernel in the counter output")
    f_fetch = CAL_BYTES / copy_f
    f_write = CAL_BYTES / copy_w
    fb = sum(t for t, _ in fetch.values()) * f_fetch / launches
    wb = sum(t for t, _ in write.values()) * f_write / launches
    label = ENTRIES[entry]
    path = os.path.join(ROOT, "profiles", "traffic.json")
    db = json.load(open(path)) if os.path.exists(path) else {}
    src = kernel_sources_hash()
    db["%s|%s" % (label, workload)] = {
        "sources": src, "bytes_per_launch": fb + wb, "fetch_bytes": fb, "write_bytes": wb,
        "fetch_factor": f_fetch, "write_factor": f_write, "calls": launches}
    json.dump(db, open(path, "w"), indent=1, sort_keys=True)
    lines = ["HBM traffic per call of %s, workload %s (kernel sources %s)" % (label, workload, src),
             "",
             "command (FETCH_SIZE pass): " + cmd_fetch,
             "command (WRITE_SIZE pass): " + cmd_write,
             "command (this summary): python3 -m delta_rule_recurrent_precond_amd.profiling "
             "record --entry %s --fetch <D1> --write <D2> --workload %s --launches %d"
             % (entry, workload, launches), "",
             "calibration: device-to-device copy of %d bytes; FETCH_SIZE reads %.6g, "
             "WRITE_SIZE reads %.6g per dispatch" % (CAL_BYTES, copy_f, copy_w),
             "scale factors (bytes per counter unit): fetch %.4f, write %.4f" % (f_fetch, f_write),
             "",
             "%-64s %9s %16s %16s" % ("kernel", "dispatches", "fetch bytes/call", "write bytes/call")]
    for n in sorted(set(fetch) | set(write)):
        tf, cf = fetch.get(n, (0.0, 0))
        tw, _ = write.get(n, (0.0, 0))
        lines.append("%-64s %9d %16.6g %16.6g" % (n[:64], cf, tf * f_fetch / launches,
                                                  tw * f_write / launches))
    lines += ["", "total bytes per call: %.6g (fetch %.6g, write %.6g)" % (fb + wb, fb, wb)]
    txt = os.path.join(ROOT, "profiles", "traffic_%s_%s.txt" % (entry, workload))
    open(txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_F32",
                 "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES")


def record_mfma(directory: str, workload: str, entry: str, launches: int, cmd: str) -> None:
    """Matrix-core work per call from one counter pass over MFMA_COUNTERS.  The
    MOPS counters count units of 512 flops.  The busy share is
    SQ_VALU_MFMA_BUSY_CYCLES / SQ_BUSY_CU_CYCLES as the counters report them: it
    counts cycles with matrix-core work in flight, so it exceeds the share of
    peak throughput that the flops alone imply."""
    per = {}
    for r in _counter_rows(directory):
        name = r.get("Kernel_Name", "")
        if not _is_library_kernel(name):
            continue
        c = r.get("Counter_Name", "").strip()
        key = (name, r.get("Dispatch_Id", r.get("Correlation_Id")))
        per.setdefault(key, {}).setdefault(c, 0.0)
        per[key][c] += float(r["Counter_Value"])
    if not per:
        raise SystemExit("no library kernel in the counter output")
    kern = {}
    for (name, _), cs in per.items():
        k = kern.setdefault(name, {"dispatches": 0, **{c: 0.0 for c in MFMA_COUNTERS}})
        k["dispatches"] += 1
        for c in MFMA_COUNTERS:
            k[c] += cs.get(c, 0.0)
    label = ENTRIES[entry]
    src = kernel_sources_hash()
    f16 = sum(k["SQ_INSTS_VALU_MFMA_MOPS_F16"] for k in kern.values()) * 512 / launches
    f32 = sum(k["SQ_INSTS_VALU_MFMA_MOPS_F32"] for k in kern.values()) * 512 / launches
    path = os.path.join(ROOT, "profiles", "mfma.json")
    db = json.load(open(path)) if os.path.exists(path) else {}
    db["%s|%s" % (label, workload)] = {"sources": src, "f16_flops_per_call": f16,
                                       "f32_flops_per_call": f32, "calls": launches}
    json.dump(db, open(path, "w"), indent=1, sort_keys=True)
    lines = ["Matrix-core work per call of %s, workload %s (kernel sources %s)" % (label, workload, src),
             "", "command (counter pass): " + cmd,
             "command (this summary): python3 -m delta_rule_recurrent_precond_amd.profiling "
             "mfma --entry %s --dir <D> --workload %s --launches %d --command <the pass's command>" % (entry, workload, launches),
             "", "MOPS counters count units of 512 flops; busy = SQ_VALU_MFMA_BUSY_CYCLES / "
             "SQ_BUSY_CU_CYCLES", "",
             "%-64s %9s %14s %14s %8s" % ("kernel", "dispatches", "f16 flop/call", "f32 flop/call",
                                          "busy")]
    for n in sorted(kern):
        k = kern[n]
        busy = k["SQ_VALU_MFMA_BUSY_CYCLES"] / k["SQ_BUSY_CU_CYCLES"] if k["SQ_BUSY_CU_CYCLES"] else 0
        lines.append("%-64s %9d %14.4g %14.4g %8.3f" % (
            n[:64], k["dispatches"], k["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512 / launches,
            k["SQ_INSTS_VALU_MFMA_MOPS_F32"] * 512 / launches, busy))
    lines += ["", "total per call: f16 %.6g flop, f32 %.6g flop" % (f16, f32)]
    txt = os.path.join(ROOT, "profiles", "mfma_%s_%s.txt" % (entry, workload))
    open(txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summary(src: str, cmd: str) -> str:
    out = ["command: " + cmd, ""]
    if src.endswith(".db"):
        c = sqlite3.connect(src)
        rows = list(c.execute(
            "select name,total_calls,total_duration,average,percentage from top_kernels"))
    else:
        rows = []
        for r in csv.DictReader(open(src)):
            rows.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]) / 1e3,
                         float(r["AverageNs"]) / 1e3, float(r["Percentage"])))
    out.append("%-110s %7s %14s %12s %7s" % ("kernel", "calls", "total_us", "avg_us", "pct"))
    for n, calls, tot, avg, pct in rows:
        out.append("%-110s %7d %14.1f %12.3f %7.2f" % (n[:110], calls, tot, avg, pct))
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python3 -m delta_rule_recurrent_precond_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    p = sub.add_parser("run")
    p.add_argument("--workload", default="1.3b-apf")
    p.add_argument("--launches", type=int, default=3)
    p.add_argument("--entry", choices=sorted(ENTRIES), required=True)
    p = sub.add_parser("record")
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--workload", default="1.3b-apf")
    p.add_argument("--launches", type=int, default=3)
    p.add_argument("--entry", choices=sorted(ENTRIES), required=True)
    p.add_argument("--cmd-fetch", default="")
    p.add_argument("--cmd-write", default="")
    p = sub.add_parser("mfma")
    p.add_argument("--dir", required=True)
    p.add_argument("--workload", default="1.3b-apf")
    p.add_argument("--launches", type=int, default=3)
    p.add_argument("--entry", choices=sorted(ENTRIES), required=True)
    p.add_argument("--command", default="")
    p = sub.add_parser("summary")
    p.add_argument("src")
    p.add_argument("--command", required=True)
    p.add_argument("--out")
    a = ap.parse_args(argv)
    if a.cmd == "run":
        run(a.workload, a.launches, a.entry)
    elif a.cmd == "record":
        record(a.fetch, a.write, a.workload, a.entry, a.launches, a.cmd_fetch, a.cmd_write)
    elif a.cmd == "mfma":
        record_mfma(a.dir, a.workload, a.entry, a.launches, a.command)
    else:
        text = summary(a.src, a.command)
        if a.out:
            open(a.out, "w").write(text)
        sys.stdout.write(text)


if __name__ == "__main__":
    main()
