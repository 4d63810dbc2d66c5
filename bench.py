"""Benchmark of the OSDN forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1.3b-apf]
                    [--no-cpu-baseline] [--only forward|phases|configs]

A step is one osdn_forward call (preconditioner walk + chunkwise pass) over
the whole workload, inputs already resident in HBM.  Several input copies
rotate so the working set exceeds the 256 MB last-level cache.  Prints ONE
JSON line (rank 0).  Besides the end-to-end figure it times the standalone
phases (osdn_precond_scan, osdn_chunk_fwd) and the plain delta rule
(OSDN_PRECOND_OFF), reports the dominant kernel against the HBM roofline,
measures every configuration (tokens/s, roofline fraction, q_geo), and times
the fp64 CPU oracle on the host as a reported baseline.  Every time is the
median of per-call HIP event times, reported with its mean, minimum and maximum.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "OSDN fwd tokens/s (scan+chunk WY), H=16 dk=dv=128 T=4096; % of roofline"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix cores, TFLOP/s
CACHE_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="1.3b-apf")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "forward", "phases", "configs"], default="all")
    return ap.parse_args()


def kernel_sources_hash() -> str:
    from delta_rule_recurrent_precond_amd.profiling import kernel_sources_hash as h
    return h()


def algorithmic_bytes(w, path: str) -> int:
    """Bytes a launch must move at minimum (inputs read once, outputs written once).

    Per token-head: q, k, v reads (dk+dk+dv elements), beta (4 B), r (4 B with
    APF), o write (dv elements); per head: S_final (dv*dk fp32) and d_final
    (dk fp32).  The two-launch chunk pass also reads k~ (dk elements) and does
    not handle r or d.
    """
    e = 2 if w.dtype == "bf16" else 4
    th = w.B * w.H * w.T
    heads = w.B * w.H
    if path == "chunk":
        per = (3 * w.dk + w.dv) * e + 4 + w.dv * e
        return th * per + heads * w.dv * w.dk * 4
    if path == "scan":
        per = w.dk * e + 4 + (4 if w.apf else 0) + w.dk * e
        return th * per + heads * w.dk * 4
    per = (2 * w.dk + w.dv) * e + 4 + (4 if w.apf else 0) + w.dv * e
    return th * per + heads * (w.dv * w.dk * 4 + w.dk * 4)


def algorithmic_flops(w) -> int:
    """Flops of one forward: per token-head the chunkwise pass (chunk form of
    the gist.science summary, §2.1: gram K K~^T, (I + A)^-1, W and U, the pseudo-
    values X, Q S^T, the scores Q K~^T and their product with X, the state
    update) is 6 dk dv + 2 C (3 dk + 2 dv) + C^2 / 3, and the preconditioner
    walk (§2.2) about 8 dk."""
    C = w.chunk
    per = 6 * w.dk * w.dv + 2 * C * (3 * w.dk + 2 * w.dv) + C * C / 3 + 8 * w.dk
    return int(w.B * w.H * w.T * per)


def _stored(name: str, kernel: str, workload: str):
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get("%s|%s" % (kernel, workload))
    except (ValueError, OSError):
        return None
    if not rec or rec.get("sources") != kernel_sources_hash():
        return None
    return rec


def stored_mfma(kernel: str, workload: str):
    """Matrix-core flops per call counted by rocprofv3 (profiles/mfma.json), if
    taken for the current kernel sources."""
    rec = _stored("mfma.json", kernel, workload)
    if rec is None:
        return None
    return {"f16_flops": rec.get("f16_flops_per_call"), "f32_flops": rec.get("f32_flops_per_call")}


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters, if they were taken
    for the current kernel sources (profiles/traffic.json)."""
    rec = _stored("traffic.json", kernel, workload)
    return rec.get("bytes_per_launch") if rec else None


def time_launches(fn, steps, warmup, torch):
    """Per-call times of fn(i): `warmup` untimed calls, then `steps` calls, each
    between two HIP events recorded on the current stream (the library launches
    on that stream), the whole run bracketed by device synchronisations.
    Returns dict(ms=median, mean, min, max, n) in milliseconds; `mean` is the
    first start to the last end over the calls."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        fn(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)
    n = len(ts)
    med = ts[n // 2] if n % 2 else 0.5 * (ts[n // 2 - 1] + ts[n // 2])
    return {"ms": med, "mean": ev[0][0].elapsed_time(ev[-1][1]) / n, "min": ts[0],
            "max": ts[-1], "n": n}


def scan_path(w, ws_bytes):
    """The launches osdn_precond_scan runs: one (walk_scan_pipe) when the
    scratch holds the flags and B*H is at most half the compute units, three
    with the scratch otherwise, else one kernel per (b,h)."""
    if not ws_bytes:
        return "single"
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return "walk_scan_pipe" if 2 * w.B * w.H <= cus else "walk_prep+walk+walk_keys"


def timing_fields(t):
    """The spread of a time_launches result, for the JSON line."""
    return {"ms": t["ms"], "ms_mean": t["mean"], "ms_min": t["min"], "ms_max": t["max"],
            "calls": t["n"]}


def cpu_baseline(w, inp):
    """The fp64 oracle on the host: the whole workload, repeated until about
    10 s of CPU time (threads x wall) have been spent."""
    from oracle import oracle
    heads = list(range(w.B * w.H))
    threads = min(oracle.default_threads(), len(heads))
    reps, wall = 0, 0.0
    while reps < 1 or (wall * threads < 10.0 and reps < 20):
        t0 = time.perf_counter()
        oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.r, eta=inp.eta, heads=heads,
                       want=("o", "S", "d"), threads=threads)
        wall += time.perf_counter() - t0
        reps += 1
    tokens = len(heads) * w.T / w.H
    return {"value": reps * tokens / wall, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "whole workload (%d (b,h) sequences x T=%d), fp64 token-serial, %d runs, "
                      "%.2f s wall on %d threads" % (len(heads), w.T, reps, wall, threads),
            "cpu_model": host_cpu_model()}


def cpu_single_thread(W):
    """The oracle on one host thread over the two smallest workloads (the tiny
    fp32 one and the 340M-style layer), tokens/s."""
    from oracle import oracle
    res = {}
    for key in ("tiny", "340m"):
        w = W.CONFIGS[key]
        inp = W.generate(w)
        t0 = time.perf_counter()
        oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.r, eta=inp.eta,
                       heads=list(range(w.B * w.H)), want=("o", "S", "d"), threads=1)
        dt = time.perf_counter() - t0
        res[key] = {"workload": w.name, "tokens_per_s": w.B * w.T / dt, "seconds": dt}
    return res


def bench_step(args, torch, osdn, W):
    """osdn_step on the decode batch: S and d updated in place each call."""
    w = W.DECODE
    dev = W.generate(w).to("cuda")
    g = torch.Generator(device="cuda").manual_seed(5)
    # enough copies of the state (S and d) that the calls rotate through at least
    # twice the 256 MB last-level cache: each call's state comes from HBM
    state_bytes = w.B * w.H * (w.dv + 1) * w.dk * 4
    copies = max(2, -(-2 * CACHE_BYTES // state_bytes))
    S = [0.1 * torch.randn(w.B, w.H, w.dv, w.dk, device="cuda", generator=g)
         for _ in range(copies)]
    d = [0.5 + torch.rand(w.B, w.H, w.dk, device="cuda", generator=g) for _ in range(copies)]
    tok = [t[:, :, 0].contiguous() for t in (dev.q, dev.k, dev.v, dev.beta, dev.r)]
    o = torch.empty_like(tok[2])
    t = time_launches(lambda i: osdn.step(tok[0], tok[1], tok[2], tok[3], S[i % copies],
                                          d[i % copies], tok[4], eta=w.eta, o=o),
                      args.steps, args.warmup, torch)
    # the same step with one state gate per key dimension
    ach = W.generate(dataclasses.replace(w, gated=True, gate_channels=True)).alpha[:, :, 0]
    ach = ach.contiguous().to("cuda")
    t_ch = time_launches(lambda i: osdn.step(tok[0], tok[1], tok[2], tok[3], S[i % copies],
                                             d[i % copies], tok[4], eta=w.eta, o=o, alpha=ach),
                         args.steps, args.warmup, torch)
    heads = w.B * w.H
    # S read and written (fp32), d read and written, q, k, v read and o written
    # (bf16), beta and r read
    nbytes = heads * (2 * w.dv * w.dk * 4 + 2 * w.dk * 4 + (2 * w.dk + 2 * w.dv) * 2 + 8)
    return {"workload": w.name, "state_copies": copies, **timing_fields(t),
            "tokens_per_s": w.B / (t["ms"] * 1e-3),
            "algorithmic_bytes": nbytes,
            "hbm_frac": nbytes / (t["ms"] * 1e-3) / (HBM_PEAK_GBS * 1e9),
            "per_channel_gate": {**timing_fields(t_ch),
                                 "hbm_frac": (nbytes + heads * w.dk * 4) / (t_ch["ms"] * 1e-3)
                                 / (HBM_PEAK_GBS * 1e9)}}


def gpu_clocks():
    """Current sclk/mclk as rocm-smi reports them (best effort, informational)."""
    import subprocess
    try:
        p = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                           text=True, timeout=20)
        card = next(iter(json.loads(p.stdout).values()))
        return {k: v for k, v in card.items() if "sclk" in k or "mclk" in k}
    except Exception:  # noqa: BLE001 - purely informational
        return None


def q_geo_of(osdn, torch, d, w, precond, ws):
    """exp of the mean of log rho_t over all (b, h, t) of one forward."""
    r = osdn.forward(d.q, d.k, d.v, d.beta, d.r, eta=d.eta, chunk=w.chunk, precond=precond,
                     workspace=ws)
    torch.cuda.synchronize()
    return float(torch.exp(r["log_ratio_sum"].double().sum() / (w.B * w.H * w.T)))


def bench_config(key, args, torch, osdn, W, steps):
    """One measured configuration: the forward on its fastest path (median of
    `steps` event-timed calls over rotating input copies), its fraction of the
    HBM roofline (algorithmic bytes), q_geo for OSDN and for the plain delta
    rule on the same inputs, and the path that ran."""
    w = W.CONFIGS[key]
    host = W.generate(w)
    per_copy = sum(t.numel() * t.element_size() for t in (host.q, host.k, host.v, host.beta))
    copies = max(2, -(-2 * CACHE_BYTES // per_copy))
    devs = [host.to("cuda") for _ in range(copies)]
    del host
    code = 0 if w.dtype == "bf16" else 1
    B, H, T, dk, dv, C = w.B, w.H, w.T, w.dk, w.dv, w.chunk
    ws_n = osdn.forward_workspace_bytes(B, H, T, dk, dv, C, code)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    path = osdn.forward_path(B, H, T, dk, dv, C, code, workspace_bytes=ws_n)
    outs = [{
        "o": torch.empty_like(d.v),
        "S_final": torch.empty((B, H, dv, dk), dtype=torch.float32, device="cuda"),
        "d_final": torch.empty((B, H, dk), dtype=torch.float32, device="cuda"),
        "log_ratio_sum": torch.empty((B, H), dtype=torch.float32, device="cuda"),
    } for d in devs]

    def fwd(i):
        d = devs[i % copies]
        osdn.forward(d.q, d.k, d.v, d.beta, d.r, eta=d.eta, chunk=C, out=outs[i % copies],
                     workspace=ws)

    t = time_launches(fwd, steps, max(3, args.warmup), torch)
    nbytes = algorithmic_bytes(w, "fused")
    res = {"workload": w.name, "path": path, **timing_fields(t),
           "tokens_per_s": B * T / (t["ms"] * 1e-3),
           "hbm_frac": nbytes / (t["ms"] * 1e-3) / (HBM_PEAK_GBS * 1e9),
           "algorithmic_bytes": nbytes,
           "q_geo": q_geo_of(osdn, torch, devs[0], w, True, ws),
           "q_geo_deltanet_mode": q_geo_of(osdn, torch, devs[0], w, False, ws)}
    if key == "tiny":
        res["note"] = "parity case (16 KB tensors): launch latency, not a roofline figure"
    del devs, outs, ws
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every (b,h) sequence is independent; see the sharding notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import delta_rule_recurrent_precond_amd as osdn
    from delta_rule_recurrent_precond_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a ROCm device"
    osdn.load()
    w = W.CONFIGS[args.workload]
    code = 0 if w.dtype == "bf16" else 1
    print("[bench] generating %s" % w.name, file=sys.stderr, flush=True)
    # the gated draw adds the state gate alpha and leaves every other input as is
    host = W.generate(dataclasses.replace(w, gated=True))
    per_copy = sum(t.numel() * t.element_size() for t in (host.q, host.k, host.v, host.beta)
                   if t is not None)
    copies = max(2, -(-2 * CACHE_BYTES // per_copy))
    devs = [host.to("cuda") for _ in range(copies)]
    B, H, T, dk, dv, C = w.B, w.H, w.T, w.dk, w.dv, w.chunk
    outs = [{
        "o": torch.empty_like(d.v),
        "S_final": torch.empty((B, H, dv, dk), dtype=torch.float32, device="cuda"),
        "d_final": torch.empty((B, H, dk), dtype=torch.float32, device="cuda"),
        "log_ratio_sum": torch.empty((B, H), dtype=torch.float32, device="cuda"),
    } for d in devs]
    ws_n = osdn.forward_workspace_bytes(B, H, T, dk, dv, C, code)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda") if ws_n else None
    path = osdn.forward_path(B, H, T, dk, dv, C, code, workspace_bytes=ws_n)

    def fpath(precond=True, single=False, per_channel=False, n=None):
        """The path osdn_forward takes for one timed variant."""
        if n is None:
            n = 0 if single else osdn.forward_workspace_bytes(B, H, T, dk, dv, C, code, precond,
                                                              per_channel=per_channel)
        return osdn.forward_path(B, H, T, dk, dv, C, code, precond, workspace_bytes=n,
                                 per_channel=per_channel)

    def fwd(i, precond=True, gated=False, single=False):
        # single: no optional scratch, so the one-kernel forward runs
        d = devs[i % copies]
        o = outs[i % copies]
        osdn.forward(d.q, d.k, d.v, d.beta, d.r, eta=d.eta, chunk=C, precond=precond,
                     alpha=d.alpha if gated else None,
                     out=o if precond else {**o, "d_final": None},
                     workspace=None if single else ws)

    print("[bench] path=%s copies=%d" % (path, copies), file=sys.stderr, flush=True)
    tf = time_launches(fwd, args.steps, args.warmup, torch)
    ms = tf["ms"]
    tokens = B * T
    result = {
        "metric": METRIC, "value": tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "timing": {"statistic": "median of per-call HIP event times", **timing_fields(tf)},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if (path in ("fused", "split") and w.dtype == "bf16") else "f32",
        "data": "synthetic (seeded generator; shapes and distributions of the workload)",
        "config": {"workload": w.name, "B": B, "H": H, "T": T, "dk": dk, "dv": dv, "chunk": C,
                   "eta": w.eta, "apf": w.apf, "storage": w.dtype, "path": path},
    }
    print("[bench] forward %.4f ms/step (median; min %.4f max %.4f)" % (ms, tf["min"], tf["max"]),
          file=sys.stderr, flush=True)

    phases = {}
    if args.only in ("all", "phases"):
        t_dn = time_launches(lambda i: fwd(i, precond=False), args.steps, args.warmup, torch)
        t_single = time_launches(lambda i: fwd(i, single=True), args.steps, args.warmup, torch)
        t_dn_single = time_launches(lambda i: fwd(i, precond=False, single=True), args.steps,
                                    args.warmup, torch)
        t_g = time_launches(lambda i: fwd(i, gated=True), args.steps, args.warmup, torch)
        t_gdn = time_launches(lambda i: fwd(i, precond=False, gated=True), args.steps,
                              args.warmup, torch)
        t_g_single = time_launches(lambda i: fwd(i, gated=True, single=True), args.steps,
                                   args.warmup, torch)
        t_gdn_single = time_launches(lambda i: fwd(i, precond=False, gated=True, single=True),
                                     args.steps, args.warmup, torch)
        # raw inputs (q, k unnormalised, beta and r as logits): the transforms done
        # inside the kernels, against separate elementwise passes before the call
        raw_host = W.generate(dataclasses.replace(w, raw=True))
        raws = [raw_host.to("cuda") for _ in range(copies)]
        del raw_host

        def fwd_raw(i, fused=True):
            d = raws[i % copies]
            o = outs[i % copies]
            if fused:
                osdn.forward(d.q, d.k, d.v, d.beta, d.r, eta=d.eta, chunk=C, out=o,
                             workspace=ws, norm_qk=True, gate_logits=True)
            else:
                qn = torch.nn.functional.normalize(d.q.float(), dim=-1).to(d.q.dtype)
                kn = torch.nn.functional.normalize(d.k.float(), dim=-1).to(d.k.dtype)
                osdn.forward(qn, kn, d.v, torch.sigmoid(d.beta),
                             None if d.r is None else torch.sigmoid(d.r), eta=d.eta, chunk=C,
                             out=o, workspace=ws)

        t_raw = time_launches(fwd_raw, args.steps, args.warmup, torch)
        t_raw_sep = time_launches(lambda i: fwd_raw(i, False), args.steps, args.warmup, torch)
        del raws
        # the per-channel gate (KDA backbone): the same draws with one gate per key
        # dimension
        kda_alpha = W.generate(dataclasses.replace(w, gated=True, gate_channels=True)).alpha
        kalphas = [kda_alpha.to("cuda") for _ in range(2)]
        del kda_alpha
        kws_n = osdn.forward_workspace_bytes(B, H, T, dk, dv, C, code, per_channel=True)
        kws = torch.empty(max(kws_n, 1), dtype=torch.uint8, device="cuda")
        kda_path = fpath(per_channel=True, n=kws_n)

        def fwd_kda(i, precond=True):
            d = devs[i % copies]
            o = outs[i % copies]
            osdn.forward(d.q, d.k, d.v, d.beta, d.r, eta=d.eta, chunk=C, precond=precond,
                         alpha=kalphas[i % 2], out=o if precond else {**o, "d_final": None},
                         workspace=kws)

        kda_steps = max(2, args.steps // 4)
        t_kda = time_launches(fwd_kda, kda_steps, 1, torch)
        t_kda_dn = time_launches(lambda i: fwd_kda(i, False), kda_steps, 1, torch)
        del kalphas, kws
        kts = [torch.empty_like(d.k) for d in devs]
        dfin = torch.empty((B, H, dk), dtype=torch.float32, device="cuda")
        lib = osdn.load()
        stream = torch.cuda.current_stream().cuda_stream

        sws_n = osdn.precond_scan_workspace_bytes(B, H, T, dk, code)
        sws = torch.empty(max(sws_n, 1), dtype=torch.uint8, device="cuda")

        def scan(i, use_ws=True):
            d = devs[i % copies]
            st = lib.osdn_precond_scan(d.k.data_ptr(), d.beta.data_ptr(),
                                       None if d.r is None else d.r.data_ptr(), None,
                                       float(d.eta), B, H, T, dk, code, kts[i % copies].data_ptr(),
                                       dfin.data_ptr(), None, None,
                                       sws.data_ptr() if (use_ws and sws_n) else None,
                                       sws_n if use_ws else 0, stream)
            assert st == 0, st

        cws_n = osdn.chunk_fwd_workspace_bytes(B, H, T, dk, dv, C, code)
        cws = torch.empty(max(cws_n, 1), dtype=torch.uint8, device="cuda")

        def chunk(i, use_ws=True):
            d = devs[i % copies]
            o = outs[i % copies]
            st = lib.osdn_chunk_fwd(d.q.data_ptr(), d.k.data_ptr(), kts[i % copies].data_ptr(),
                                    d.v.data_ptr(), d.beta.data_ptr(), None, None, B, H, T, dk,
                                    dv, C,
                                    code, 0, o["o"].data_ptr(), o["S_final"].data_ptr(),
                                    cws.data_ptr() if (use_ws and cws_n) else None,
                                    cws_n if use_ws else 0, stream)
            assert st == 0, st

        t_scan = time_launches(scan, args.steps, args.warmup, torch)
        t_scan_single = time_launches(lambda i: scan(i, False), args.steps, args.warmup, torch)
        t_chunk = time_launches(chunk, args.steps, args.warmup, torch)
        t_chunk_single = time_launches(lambda i: chunk(i, False), args.steps, args.warmup, torch)
        ms_dn, ms_scan, ms_chunk = t_dn["ms"], t_scan["ms"], t_chunk["ms"]
        ms_g, ms_gdn = t_g["ms"], t_gdn["ms"]

        def entry(t, p, **kw):
            return {**timing_fields(t), "tokens_per_s": tokens / (t["ms"] * 1e-3), "path": p,
                    **kw}

        phases = {
            "forward_single_kernel": entry(t_single, fpath(single=True),
                                           traffic=stored_traffic("osdn_fused_forward",
                                                                  args.workload)),
            "deltanet_mode_single_kernel": entry(t_dn_single, fpath(False, single=True)),
            "precond_scan": entry(t_scan, scan_path(w, sws_n),
                                  hbm_frac=algorithmic_bytes(w, "scan") / (ms_scan * 1e-3)
                                  / (HBM_PEAK_GBS * 1e9),
                                  traffic=stored_traffic("osdn_precond_scan_split",
                                                         args.workload)),
            "precond_scan_single_kernel": entry(t_scan_single, "one kernel per (b,h)"),
            "chunk_fwd": entry(t_chunk, "chunk_prep+chunk_state" if cws_n else "single",
                               hbm_frac=algorithmic_bytes(w, "chunk") / (ms_chunk * 1e-3)
                               / (HBM_PEAK_GBS * 1e9),
                               traffic=stored_traffic("osdn_chunk_fwd_split", args.workload)),
            "chunk_fwd_single_kernel": entry(t_chunk_single, "single fused kernel (given kt)"),
            "deltanet_mode": entry(t_dn, fpath(False),
                                   traffic=stored_traffic("osdn_deltanet_split", args.workload)),
            "precond_overhead": (ms - ms_dn) / ms,
            "gated_forward": entry(t_g, fpath(), vs_ungated=ms_g / ms,
                                   traffic=stored_traffic("osdn_forward_gated_split",
                                                          args.workload)),
            "gated_deltanet_mode": entry(t_gdn, fpath(False)),
            "gated_forward_single_kernel": entry(t_g_single, fpath(single=True)),
            "gated_deltanet_mode_single_kernel": entry(t_gdn_single, fpath(False, single=True)),
            "gated_precond_overhead": (ms_g - ms_gdn) / ms_g,
            "raw_inputs_transforms_in_kernels": entry(
                t_raw, fpath(), traffic=stored_traffic("osdn_forward_raw_split", args.workload)),
            "per_channel_gate_forward": entry(t_kda, kda_path,
                                              traffic=stored_traffic("osdn_forward_kda_split",
                                                                     args.workload)),
            "per_channel_gate_deltanet_mode": entry(t_kda_dn, fpath(False, per_channel=True)),
            "raw_inputs_separate_torch_passes": entry(t_raw_sep, fpath()),
            "two_launch_scan_share": ms_scan / (ms_scan + ms_chunk),
        }
        result["phases"] = phases
        print("[bench] scan %.4f ms, chunk %.4f ms, deltanet %.4f ms" % (ms_scan, ms_chunk, ms_dn),
              file=sys.stderr, flush=True)

    # Against the HBM roofline.  On the matrix-core shapes the unit is one
    # osdn_forward call: the single fused kernel, or the pipeline of launches
    # (the walk with its preparation, chunk_prep, chunk_state) timed as one call
    # on its stream,
    # with the method's algorithmic bytes (q, k, v, beta, r in; o out).  The
    # two-launch path is dominated by the chunkwise pass.
    if path == "split":
        kname, kms, kbytes = "osdn_forward_split", ms, algorithmic_bytes(w, "fused")
    elif path == "fused":
        kname, kms, kbytes = "osdn_fused_forward", ms, algorithmic_bytes(w, "fused")
    else:
        kname = "chunk_generic"
        kms = phases["chunk_fwd"]["ms"] if phases else ms
        kbytes = algorithmic_bytes(w, "chunk")
    achieved = kbytes / (kms * 1e-3) / 1e9
    result["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                          "traffic": stored_traffic(kname, args.workload),
                          "kernel": kname, "algorithmic_bytes": kbytes, "kernel_ms": kms}
    # the same call against the matrix cores: the method's flops over the time,
    # beside what the counters saw the matrix cores do (fp16 operands)
    flops = algorithmic_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    result["mfma"] = {"achieved": tflops, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": tflops / MFMA_PEAK_TFLOPS, "algorithmic_flops": flops,
                      "operands": "fp16, fp32 accumulation",
                      "counters": stored_mfma(kname, args.workload)}
    # geometric mean of the residual ratios rho_t over all (b, h, t), OSDN and
    # the plain delta rule on the same inputs
    result["q_geo"] = {"osdn": q_geo_of(osdn, torch, devs[0], w, True, ws),
                       "deltanet_mode": q_geo_of(osdn, torch, devs[0], w, False, ws)}

    if args.only in ("all", "phases"):
        result["decode_step"] = bench_step(args, torch, osdn, W)

    if args.only in ("all", "configs"):
        # every measured configuration on its fastest path (the metric one above
        # included, re-timed in the same way)
        del devs, outs, ws
        torch.cuda.empty_cache()
        cfg = {}
        for key in ("tiny", "340m", "340m-apf", "1.3b-apf", "recall", "recall-apf"):
            print("[bench] config %s" % key, file=sys.stderr, flush=True)
            cfg[key] = bench_config(key, args, torch, osdn, W, max(20, args.steps // 2))
        result["configs"] = cfg

    result["gpu_clocks"] = gpu_clocks()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, host)
        result["cpu_single_thread"] = cpu_single_thread(W)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
