#!/usr/bin/env python
"""Benchmark of the decode MoE layer with batch-aware expert selection on one
MI355X: layer latency, active-expert count and expert-weight HBM bandwidth.

One step = one moe_layer_decode call (router, selection, gate weights,
compaction, grouped SwiGLU FFN) over one batch of seeded synthetic tokens.
Steps are replayed from HIP graphs, each chaining R steps over R
bit-identical copies of the weights at different addresses, so the 256 MB
Infinity Cache cannot serve the active experts from one step to the next.
Inputs are resident in HBM before the timed region starts. Percentiles are
over graph replays (per-step averages within one replay).

Prints one JSON line (rank 0, N = 1). `value` is the active-expert weight
bytes of one step divided by the measured step time (GB/s).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
KERNEL_SOURCES = ("aware_expert_routing_amd/csrc/ffn.hip", "aware_expert_routing_amd/csrc/moe_internal.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_kernel_qwen3_30b_B16_oea4_traffic.json")
METRIC = "MoE-layer decode µs + expert-weight HBM GB/s (% of peak), B=16, E=128 k=8"


def _parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="qwen3_30b_bf16")
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--policy", default="oea", choices=["topk", "oea", "budget", "greedy", "hier", "lynx"])
    ap.add_argument("--k0", type=int, default=4)
    ap.add_argument("--m", type=int, default=32)
    ap.add_argument("--g", type=int, default=4, help="hier: tokens per request (--k0 is the request budget)")
    ap.add_argument("--rotate-bytes", type=float, default=2.0e9,
                    help="replicas are added until they hold this many distinct active bytes")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle time with all threads (half of it again with 1 thread)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", default=None,
                    help="run every configured (config, B, policy) case; one JSON line each to this file")
    ap.add_argument("--sweep-policies", default=None, metavar="P1,P2",
                    help="with --sweep: only these policies (e.g. greedy,hier)")
    ap.add_argument("--ffn-only", type=int, default=0, metavar="N",
                    help="run N eager moe_expert_ffn calls on rotating replicas and exit (for counter runs)")
    ap.add_argument("--read-ceiling", type=float, default=0.0, metavar="MB",
                    help="time a read-only reduction over MB megabytes (8 rotating buffers) and exit: "
                         "the achievable HBM read rate on this GPU")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="MB",
                    help="run a plain device copy of MB megabytes 10 times and exit (counter scale)")
    ap.add_argument("--phase-timeline", type=int, default=0, metavar="N",
                    help="load the measurement library (expert FFN with phase stamps) and print, over N "
                         "launches on rotating replicas, when each phase ends (p50 and max over "
                         "workgroups, median over launches) and the weight bytes consumed per microsecond")
    ap.add_argument("--write-traffic", default=None, metavar="DIR",
                    help="no GPU: read the rocprofv3 counter CSVs of four passes under DIR (copy_fetch, "
                         "copy_write, ffn_fetch, ffn_write; the copy of --copy-calibration MB and "
                         "--ffn-only launches of the chosen workload) and write the traffic summary "
                         "that the roofline's `traffic` field reads")
    return ap.parse_args()


def _percentiles(v):
    v = np.sort(np.asarray(v))
    return float(np.median(v)), float(np.percentile(v, 10)), float(np.percentile(v, 90))


class Case:
    """Device state for one (config, B, policy) workload."""

    def __init__(self, cfg, B, policy, k0, m, inp, dev_base, rotate_bytes, g=0):
        import torch
        from aware_expert_routing_amd import _lib as L

        self.cfg, self.B = cfg, B
        self.policy = L.make_policy(policy, cfg.k, k0, m, g)
        self.policy_name = policy
        self.k0, self.m = k0, m
        tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self.x = dev_base["x"][:B].contiguous()
        self.bias = dev_base["bias"]
        self.ws = L.alloc_workspace(B, cfg.d, cfg.E, cfg.I, cfg.k, tdt)
        self.logits = torch.empty((B, cfg.E), dtype=torch.float32, device="cuda")
        self.routing = L.Routing(B, cfg.E, cfg.k)
        self.y = torch.empty((B, cfg.d), dtype=tdt, device="cuda")
        # One eager call to learn the active set.
        L.moe_layer_decode(self.x, dev_base["w_g"], self.bias, dev_base["w_gate"], dev_base["w_up"],
                           dev_base["w_down"], self.policy, self.logits, self.routing, self.y, self.ws)
        torch.cuda.synchronize()
        self.n_active = int(self.routing.n_active.item())
        self.active_bytes = self.n_active * cfg.expert_bytes
        self.pairs = int(self.routing.expert_offsets[self.n_active].item())
        reps = max(2, math.ceil(rotate_bytes / max(1, self.active_bytes)))
        pool = cfg.E * cfg.expert_bytes
        reps = min(reps, max(2, int(48e9 // pool)))
        self.replicas = [dev_base] + [{k: (v.clone() if k in ("w_g", "w_gate", "w_up", "w_down") else v)
                                       for k, v in dev_base.items()} for _ in range(reps - 1)]
        self.L = L

    def layer(self, rep):
        d = self.replicas[rep]
        self.L.moe_layer_decode(self.x, d["w_g"], self.bias, d["w_gate"], d["w_up"], d["w_down"],
                                self.policy, self.logits, self.routing, self.y, self.ws)

    def ffn(self, rep, lib=None):
        d = self.replicas[rep]
        self.L.moe_expert_ffn(self.x, d["w_gate"], d["w_up"], d["w_down"], self.routing, self.y, self.ws,
                              lib=lib)


def _capture_chain(fn, first, count):
    """One HIP graph of `count` consecutive calls fn(first), fn(first+1), ...
    (each on its own weight replica)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in range(first, first + count):
            fn(r)
    return g


def _time_steps(fn, R, steps, warmup):
    """Times exactly `steps` calls of fn, replayed from graphs that chain R
    calls (one per replica) plus one tail graph, with events recorded on the
    replay stream between graph launches. Returns per-call times (ms) of each
    replay and the total over the timed region."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for r in range(R):  # warm the code paths outside capture
            fn(r)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    full = _capture_chain(fn, 0, R)
    n_full, tail_n = divmod(steps, R)
    tail = _capture_chain(fn, 0, tail_n) if tail_n else None
    torch.cuda.synchronize()
    for _ in range(max(1, warmup // R)):
        full.replay()
    torch.cuda.synchronize()
    plan = [(full, R)] * n_full + ([(tail, tail_n)] if tail else [])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(plan) + 1)]
    ev[0].record()
    for i, (g, _) in enumerate(plan):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) / n for i, (_, n) in enumerate(plan)]
    total = ev[0].elapsed_time(ev[-1])
    del full, tail
    return per, total


def _kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _traffic(workload):
    """HBM bytes per launch of the FFN kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by a plain copy of known
    size), or None when there is none for this workload or the kernel
    sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != _kernel_source_hash() or t.get("workload") != workload:
        return None
    return int(t["fetch_bytes"] + t["write_bytes"])


def _counter_mean(dirpath, counter, kernel_substr):
    """Mean per dispatch of one counter over the dispatches of kernels whose
    name contains kernel_substr, from the rocprofv3 CSVs under dirpath."""
    import csv
    import glob
    vals = []
    for path in glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") == counter and kernel_substr in row.get("Kernel_Name", ""):
                    vals.append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel_substr!r} under {dirpath}")
    return float(np.mean(vals)), len(vals)


def _write_traffic(dirpath, workload, copy_bytes, active_bytes):
    """Traffic summary of the FFN kernel: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) scaled by what the same counters read for a plain copy that
    reads and writes copy_bytes."""
    cf, _ = _counter_mean(os.path.join(dirpath, "copy_fetch"), "FETCH_SIZE", "copyBuffer")
    cw, _ = _counter_mean(os.path.join(dirpath, "copy_write"), "WRITE_SIZE", "copyBuffer")
    ff, nf = _counter_mean(os.path.join(dirpath, "ffn_fetch"), "FETCH_SIZE", "ffn_kernel")
    fw, nw = _counter_mean(os.path.join(dirpath, "ffn_write"), "WRITE_SIZE", "ffn_kernel")
    sf, sw = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    out = {"workload": workload, "kernel": "ffn_kernel", "source_sha256": _kernel_source_hash(),
           "fetch_bytes": int(round(ff * 1024.0 * sf)), "write_bytes": int(round(fw * 1024.0 * sw)),
           "fetch_size_kib_per_dispatch": ff, "write_size_kib_per_dispatch": fw,
           "dispatches": [nf, nw], "copy_scale_fetch": sf, "copy_scale_write": sw,
           "algorithmic_bytes": active_bytes}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


PHASES = ["start", "routing lists in LDS", "first stage computed", "gate/up done", "first grid barrier passed",
          "first down stages landed", "last down stage computed", "down rows stored", "rows counted",
          "combine done", "end"]


def _phase_timeline(c, launches):
    """Phase ends of the expert FFN from the measurement library's stamps
    (100 MHz clock, relative to the first workgroup's start), and the weight
    bytes consumed per 1-us bin (32 KB of weights per stage)."""
    import ctypes
    import torch
    from aware_expert_routing_amd import build as B
    lib = c.L.load(B.PHASES_LIB)
    lib.moe_phase_stamps.argtypes = [ctypes.c_void_p]
    st = torch.zeros(256 * 64, dtype=torch.int64, device="cuda")
    R = len(c.replicas)
    for i in range(R):
        c.ffn(i, lib=lib)
    torch.cuda.synchronize()
    lib.moe_phase_stamps(st.data_ptr())
    runs = []
    for i in range(launches):
        st.zero_()
        c.ffn((i * 7) % R, lib=lib)
        torch.cuda.synchronize()
        raw = st.view(256, 64).cpu().numpy().view(np.uint64)
        used = raw[:, 0] > 0
        raw = raw[used]
        t0 = float(raw[:, 0].min())
        t = (raw & np.uint64((1 << 63) - 1)).astype(np.float64)
        runs.append(np.where(t > 0, (t - t0) * 0.01, np.nan))
    lib.moe_phase_stamps(None)
    torch.cuda.synchronize()
    rows = []
    for i, name in enumerate(PHASES):
        col = [r[:, i] for r in runs]
        n = int(np.median([np.isfinite(v).sum() for v in col]))
        p50 = float(np.median([np.nanmedian(v) for v in col if np.isfinite(v).any()]))
        mx = float(np.median([np.nanmax(v) for v in col if np.isfinite(v).any()]))
        rows.append({"phase": name, "p50_us": round(p50, 2), "max_us": round(mx, 2), "workgroups": n})
    stages = np.concatenate([r[:, 16:64].ravel() for r in runs])
    stages = stages[np.isfinite(stages)]
    hist = np.bincount(stages.astype(int)) * 32768 / len(runs) / 1e3  # GB/s in each 1-us bin
    return {"phases": rows, "weight_GBps_per_us": [round(float(v)) for v in hist], "launches": launches}


def _cpu_threads():
    """Host threads for the oracle: the CPUs this process may run on, capped
    by OMP_NUM_THREADS when the environment sets it (a shared host's CPU
    share)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return n


def _time_oracle(args, kw, seconds, threads):
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import moe_oracle as orc

    times = []
    with threadpool_limits(limits=threads):
        used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        t_end = time.perf_counter() + seconds
        while True:
            t0 = time.perf_counter()
            orc.moe_layer(*args, **kw)
            times.append(time.perf_counter() - t0)
            if (time.perf_counter() > t_end and len(times) >= 5) or len(times) >= 200:
                break
    return float(np.median(times)), len(times), int(used)


def _cpu_baseline(cfg, inp, B, policy, k0, m, active_bytes, seconds, g=0):
    args = (inp["x"][:B], inp["w_g"], inp["bias"], inp["w_gate"], inp["w_up"], inp["w_down"],
            cfg.dtype, policy, cfg.k, k0, m)
    kw = {"g": g}
    affinity = len(os.sched_getaffinity(0))
    med, n, used = _time_oracle(args, kw, seconds, _cpu_threads())
    med1, n1, _ = _time_oracle(args, kw, seconds / 2, 1)
    return {"value": active_bytes / med / 1e9, "unit": "GB/s", "cores": used, "kind": "oracle",
            "cores_available": affinity,
            "value_1_thread": active_bytes / med1 / 1e9,
            "sample": f"{n} full oracle layer calls with {used} BLAS threads and {n1} with 1 thread "
                      f"(numpy float64: router, selection, SwiGLU over the active experts with bf16 "
                      f"widening) on the same B={B} batch; median {med * 1e3:.1f} ms per call "
                      f"({med1 * 1e3:.1f} ms with 1 thread)"}


def _policy_name(policy, k0, m, g):
    return policy + {"oea": f"(k0={k0})", "budget": f"(m={m})", "greedy": f"(m={m})",
                     "hier": f"(m={m},m_r={k0},g={g})", "lynx": f"(m={m})"}.get(policy, "")


def _run_case(cfg, B, policy, k0, m, inp, dev, args, with_cpu, g=0):
    import torch

    c = Case(cfg, B, policy, k0, m, inp, dev, args.rotate_bytes, g)
    R = len(c.replicas)
    per, total = _time_steps(c.layer, R, args.steps, args.warmup)
    med, p10, p90 = _percentiles(per)
    ms_per_step = total / args.steps
    # The expert FFN alone (one kernel for bf16): its average launch time.
    _, total_f = _time_steps(c.ffn, R, args.steps, args.warmup)
    ffn_ms = total_f / args.steps
    # Every timed call shared this workspace: a grid-wide wait that gave up
    # would have left its outputs unspecified.
    c.L.check_workspace(c.ws)
    value = c.active_bytes / (ms_per_step * 1e-3) / 1e9
    ffn_gbps = c.active_bytes / (ffn_ms * 1e-3) / 1e9
    pol = _policy_name(policy, k0, m, g)
    out_workload = (f"{cfg.name} decode MoE layer, B={B}, d={cfg.d}, E={cfg.E}, k={cfg.k}, "
                    f"I={cfg.I}, policy {pol}")
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; shapes and distributions of the named layer)",
        "config": {"workload": out_workload,
                   "batch": B, "policy": pol, "replicas": R},
        "layer_us": {"median": round(med * 1e3, 2), "p10": round(p10 * 1e3, 2),
                     "p90": round(p90 * 1e3, 2), "mean": round(ms_per_step * 1e3, 2),
                     "samples": len(per), "steps_per_sample": R,
                     "note": "percentiles over graph replays, each the mean of its chained steps"},
        "n_active": c.n_active,
        "pairs": c.pairs,
        "active_expert_bytes": c.active_bytes,
        "pct_of_hbm_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "expert_ffn_us": round(ffn_ms * 1e3, 2),
        "roofline": {"bound": "hbm", "achieved": round(ffn_gbps, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(ffn_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": _traffic(out_workload),
                     "kernel": "ffn_kernel (moe_expert_ffn: gate/up, SwiGLU, down and combine, one launch)",
                     "bytes_per_launch": c.active_bytes},
    }
    if with_cpu:
        out["cpu_baseline"] = _cpu_baseline(cfg, inp, B, policy, k0, m, c.active_bytes, args.cpu_seconds, g)
    del c
    torch.cuda.empty_cache()
    return out


def _upload(inp, dtype):
    import torch

    def up(a):
        if a is None:
            return None
        if dtype == "bf16" and a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return {k: up(v) for k, v in inp.items()}


def main():
    args = _parse()
    if args.write_traffic:
        from aware_expert_routing_amd.workloads import CONFIGS
        cfg = CONFIGS[args.config]
        # The active set is the one the GPU run found: taken from the counter
        # pass's own printout (bench.py --ffn-only), saved beside the CSVs.
        with open(os.path.join(args.write_traffic, "ffn_only.json")) as f:
            info = json.loads([ln for ln in f.read().splitlines() if ln.startswith('{"ffn_launches"')][-1])
        pol = _policy_name(args.policy, args.k0, args.m, args.g)
        workload = (f"{cfg.name} decode MoE layer, B={args.batch}, d={cfg.d}, E={cfg.E}, k={cfg.k}, "
                    f"I={cfg.I}, policy {pol}")
        _write_traffic(args.write_traffic, workload, int(args.copy_calibration * 1e6) // 4 * 4,
                       info["active_expert_bytes"])
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: there is no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    from aware_expert_routing_amd.workloads import CONFIGS, make_layer

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.read_ceiling:
        # Eight distinct buffers in rotation, so the 256 MB Infinity Cache
        # cannot serve one reduction from the previous one.
        from aware_expert_routing_amd import _lib as L
        n = int(args.read_ceiling * 1e6) // 16 * 4
        bufs = [torch.ones(n, dtype=torch.float32, device="cuda") for _ in range(8)]
        out = torch.empty((), dtype=torch.float32, device="cuda")
        words = torch.empty(1024, dtype=torch.int32, device="cuda")
        reps = 40
        for name, fn in (("moe_read_stream (16-byte loads, 1024 workgroups)",
                          lambda b: L.moe_read_stream(b, words)),
                         ("torch.sum (read-only reduction)", lambda b: torch.sum(b, dim=0, out=out))):
            for b in bufs:
                fn(b)
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            ev0.record()
            for i in range(reps):
                fn(bufs[i % 8])
            ev1.record()
            torch.cuda.synchronize()
            ms = ev0.elapsed_time(ev1) / reps
            print(json.dumps({"read_only_bytes": n * 4, "us_per_pass": round(ms * 1e3, 2),
                              "read_GBps": round(n * 4 / (ms * 1e-3) / 1e9, 1), "passes": reps,
                              "kernel": name}))
        return
    if args.copy_calibration:
        n = int(args.copy_calibration * 1e6) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 10}))
        return
    if args.sweep:
        with open(args.sweep, "w") as f:
            for cname, cfg in CONFIGS.items():
                inp = make_layer(cfg, max(cfg.batches))
                dev = _upload(inp, cfg.dtype)
                pols = [("topk", 0, 0, 0)] + [("oea", k0, 0, 0) for k0 in cfg.oea_k0] + \
                       [("budget", 0, m, 0) for m in cfg.budget_m] + \
                       [("greedy", 0, m, 0) for m in cfg.budget_m]
                if cname == "specdec_bf16":  # requests of 4 drafts
                    pols += [("hier", m // 4, m, 4) for m in cfg.budget_m]
                if cname in ("qwen3_30b_bf16", "lynx_bf16"):
                    pols += [("lynx", 0, m, 0) for m in cfg.budget_m if m >= cfg.k]
                if args.sweep_policies:
                    keep = set(args.sweep_policies.split(","))
                    pols = [p for p in pols if p[0] in keep]
                for B in cfg.batches:
                    for pol, k0, m, g in pols:
                        rec = _run_case(cfg, B, pol, k0, m, inp, dev, args, with_cpu=False, g=g)
                        f.write(json.dumps(rec) + "\n")
                        f.flush()
                        print(f"{cname} B={B} {pol}{k0 or m or ''}: n_active={rec['n_active']} "
                              f"layer {rec['layer_us']['median']} us, {rec['value']} GB/s, "
                              f"ffn {rec['roofline']['achieved']} GB/s", flush=True)
                del dev
                torch.cuda.empty_cache()
        return
    cfg = CONFIGS[args.config]
    inp = make_layer(cfg, max(args.batch, max(cfg.batches)))
    dev = _upload(inp, cfg.dtype)
    if args.phase_timeline:
        c = Case(cfg, args.batch, args.policy, args.k0, args.m, inp, dev, args.rotate_bytes,
                 args.g if args.policy == "hier" else 0)
        tl = _phase_timeline(c, args.phase_timeline)
        for r in tl["phases"]:
            print(f"{r['phase']:28s} p50 {r['p50_us']:7.2f} us  max {r['max_us']:7.2f} us  ({r['workgroups']} workgroups)")
        print("weight GB/s consumed per 1-us bin:", " ".join(f"{i}:{v}" for i, v in enumerate(tl["weight_GBps_per_us"])))
        print(json.dumps({"n_active": c.n_active, "active_expert_bytes": c.active_bytes, **tl}), flush=True)
        return
    if args.ffn_only:
        c = Case(cfg, args.batch, args.policy, args.k0, args.m, inp, dev, args.rotate_bytes,
                 args.g if args.policy == "hier" else 0)
        for i in range(args.ffn_only):
            c.ffn(i % len(c.replicas))
        torch.cuda.synchronize()
        print(json.dumps({"ffn_launches": args.ffn_only, "n_active": c.n_active,
                          "active_expert_bytes": c.active_bytes}), flush=True)
        return
    rec = _run_case(cfg, args.batch, args.policy, args.k0, args.m, inp, dev, args,
                    with_cpu=not args.no_cpu_baseline, g=args.g if args.policy == "hier" else 0)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
