"""Measured HBM traffic and kernel-time summaries for the library's kernels.

HBM bytes per launch come from two rocprofv3 counter passes over the same
program (the counter blocks cannot hold FETCH_SIZE and WRITE_SIZE in one pass),
each scaled by what the same counter reads for a device-to-device copy of a
known size run in the same process:

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d D1 -o run -- \\
        python3 -m delta_rule_recurrent_precond_amd.profiling run
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d D2 -o run -- \\
        python3 -m delta_rule_recurrent_precond_amd.profiling run
    python3 -m delta_rule_recurrent_precond_amd.profiling record --fetch D1 --write D2

`record` writes profiles/traffic.json (read by bench.py; an entry only counts
while the kernel sources are unchanged) and a text summary under profiles/.
`summary` turns a rocprofv3 --kernel-trace --stats output (kernel_stats.csv or
the SQLite database) into the text tables kept under profiles/.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CAL_BYTES = 1 << 30  # calibration copy: 1 GiB read, 1 GiB written
# template argument of osdn_fused_forward -> the entry point it serves
MODES = {"0": "osdn_fused_forward", "1": "osdn_fused_deltanet", "2": "osdn_fused_chunk",
         "3": "osdn_fused_scan"}


def kernel_sources_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "delta_rule_recurrent_precond_amd", "csrc", "*"))):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def _kernel_label(name: str):
    """Entry-point label of an osdn kernel name (mangled or demangled), or None."""
    if "osdn_fused_forward" not in name:
        return None
    for key, label in MODES.items():
        if "ILi%sE" % key in name or "osdn_fused_forward<%s>" % key in name:
            return label
    return None


def run(workload: str, launches: int) -> None:
    """The program the counter passes profile: a calibration copy, then
    `launches` calls of each fused entry point on the workload."""
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
    w = W.CONFIGS[workload]
    dev = W.generate(w).to("cuda")
    for _ in range(launches):
        osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, eta=dev.eta, chunk=w.chunk)
        osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, eta=dev.eta, chunk=w.chunk,
                     precond=False)
        sc = osdn.precond_scan(dev.k, dev.beta, dev.r, None, dev.eta)
        osdn.chunk_fwd(dev.q, dev.k, sc["k_tilde"], dev.v, dev.beta, chunk=w.chunk)
    torch.cuda.synchronize()
    print("profiled program done: %s, %d launches per entry point" % (workload, launches),
          flush=True)


def _counter_rows(directory: str):
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % directory)
    rows = []
    for f in files:
        for r in csv.DictReader(open(f)):
            rows.append(r)
    return rows


def _means(directory: str, counter: str):
    """Mean counter value per dispatch for the calibration copy and each osdn kernel."""
    sums, counts = {}, {}
    for r in _counter_rows(directory):
        if r.get("Counter_Name", "").strip() != counter:
            continue
        name = r.get("Kernel_Name", "")
        label = _kernel_label(name)
        if label is None and "copy" in name.lower():
            label = "copy"
        if label is None:
            continue
        v = float(r["Counter_Value"])
        # one row per dispatch and counter (values already summed over instances)
        key = (label, r.get("Dispatch_Id", r.get("Correlation_Id")))
        sums[key] = sums.get(key, 0.0) + v
    per = {}
    for (label, _), v in sums.items():
        per.setdefault(label, []).append(v)
    out = {}
    for label, vs in per.items():
        if label == "copy":
            vs = sorted(vs)[-3:]  # the three 1 GiB copies are the largest
        out[label] = (sum(vs) / len(vs), len(vs))
    return out


def record(fetch_dir: str, write_dir: str, workload: str, cmd_fetch: str, cmd_write: str) -> None:
    fetch = _means(fetch_dir, "FETCH_SIZE")
    write = _means(write_dir, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("calibration copy not found in the counter output")
    f_fetch = CAL_BYTES / fetch["copy"][0]
    f_write = CAL_BYTES / write["copy"][0]
    path = os.path.join(ROOT, "profiles", "traffic.json")
    db = json.load(open(path)) if os.path.exists(path) else {}
    src = kernel_sources_hash()
    lines = ["HBM traffic per launch, workload %s (kernel sources %s)" % (workload, src), "",
             "command (FETCH_SIZE pass): " + cmd_fetch,
             "command (WRITE_SIZE pass): " + cmd_write,
             "command (this summary): python3 -m delta_rule_recurrent_precond_amd.profiling "
             "record --fetch <D1> --write <D2> --workload %s" % workload, "",
             "calibration: device-to-device copy of %d bytes; FETCH_SIZE reads %.6g, "
             "WRITE_SIZE reads %.6g per dispatch" % (CAL_BYTES, fetch["copy"][0], write["copy"][0]),
             "scale factors (bytes per counter unit): fetch %.4f, write %.4f" % (f_fetch, f_write),
             "",
             "%-22s %9s %14s %14s %16s" % ("kernel", "launches", "FETCH_SIZE", "WRITE_SIZE",
                                          "bytes/launch")]
    for label in MODES.values():
        if label not in fetch or label not in write:
            continue
        fb = fetch[label][0] * f_fetch
        wb = write[label][0] * f_write
        db["%s|%s" % (label, workload)] = {
            "sources": src, "bytes_per_launch": fb + wb, "fetch_bytes": fb, "write_bytes": wb,
            "fetch_factor": f_fetch, "write_factor": f_write}
        lines.append("%-22s %9d %14.6g %14.6g %16.6g" % (label, fetch[label][1], fetch[label][0],
                                                         write[label][0], fb + wb))
    json.dump(db, open(path, "w"), indent=1, sort_keys=True)
    txt = os.path.join(ROOT, "profiles", "traffic_fused_kernels_%s.txt" % workload)
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
    p = sub.add_parser("record")
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--workload", default="1.3b-apf")
    p.add_argument("--cmd-fetch", default="")
    p.add_argument("--cmd-write", default="")
    p = sub.add_parser("summary")
    p.add_argument("src")
    p.add_argument("--command", required=True)
    p.add_argument("--out")
    a = ap.parse_args(argv)
    if a.cmd == "run":
        run(a.workload, a.launches)
    elif a.cmd == "record":
        record(a.fetch, a.write, a.workload, a.cmd_fetch, a.cmd_write)
    else:
        text = summary(a.src, a.command)
        if a.out:
            open(a.out, "w").write(text)
        sys.stdout.write(text)


if __name__ == "__main__":
    main()
