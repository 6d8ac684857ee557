#!/usr/bin/env python3
"""Benchmark of the VC-Attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic
Wan2.2-720p-shaped input (B=1, H=40, S=75600 = 21x45x80, D=128), inputs
resident in HBM:  vc_quantize(Q) -> vc_smooth_group(K, V: 64-cluster k-means,
4 iterations, argsort, K/V permute, block means, E4M3 residuals) ->
vc_attn_fwd (FP8 matrix cores, ExpCast codes, mean restoration, mid-window
key order).

Reported `value` is the metric the workload is quoted on: vc_attn_fwd
TFLOP/s (4*S^2*D*H algorithmic flops over the attention kernel's duration,
HIP events on the stream it runs on), with `roofline` against the published
dense FP8 matrix-core peak; `ms_per_step` is the whole path.  The CPU oracle
is timed on a bounded sample of the same workload (`cpu_baseline`), and the
in-house BF16 baseline on the same kernel skeleton gives the speedup.

Usage: python bench.py [--gpus 1] [--steps 5] [--warmup 2] [--workload wan]
       python bench.py --traffic-job          (under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)
       python bench.py --traffic-summary FETCH_DIR WRITE_DIR OUT_JSON COMMAND
       python bench.py --prep-job [--workload minimax]   (the preparation passes, for --pmc runs)
       python bench.py --counter-summary OUT_MD TITLE DIR [DIR ...]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0   # MI355X published dense FP8 matrix-core peak
BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense BF16 matrix-core peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fp8_wan_traffic.json")
# the attention kernel's sources: its file and the header of shared device helpers
ATTN_SRC = [os.path.join(ROOT, "bit_fp8_attention_amd", "csrc", f) for f in ("vc_attn_fp8.hip", "vc_common.hpp")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _sha(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_profile():
    """HBM bytes per launch of the attention kernel from the committed
    rocprofv3 counter summary, or None when the kernel has changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != _sha(ATTN_SRC):
        return None
    return t.get("bytes_per_launch")


COPY_BYTES = 1 << 30  # calibration copy: reads and writes exactly this many bytes


def traffic_job(w):
    """One V-Smooth attention launch on the workload, then one plain device
    copy of COPY_BYTES as the very last dispatch.  Meant to run under
    `rocprofv3 --pmc FETCH_SIZE` (then WRITE_SIZE); `--traffic-summary` turns
    the two runs into HBM bytes per attention launch, scaled by what the same
    counter reads for the copy of known size."""
    import torch

    import bit_fp8_attention_amd as vc
    import vcsynth
    q, k, v = vcsynth.make_qkv(w.name, device="cuda")
    qz = vc.vc_quantize(q, sm_scale=w.sm_scale)
    g = vc.vc_smooth_group(k, v, w.clusters, w.iters, w.seed)
    o = torch.empty_like(q)
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    vc.vc_attn_fwd(qz["q8"], qz["q_scale"], g["k8"], g["k_scale"], g["r8"], g["r_scale"], g["mu_split"], S=w.S,
                   out=o)
    b.copy_(a)
    torch.cuda.synchronize()
    log("traffic job done")


def _counter_rows(d, counter):
    import csv
    import glob
    rows = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                did = int(r["Dispatch_Id"])
                name, val = rows.get(did, (r["Kernel_Name"], 0.0))
                rows[did] = (name, val + float(r["Counter_Value"]))
    if not rows:
        raise SystemExit(f"no {counter} rows under {d}")
    return rows


def traffic_summary(fetch_dir, write_dir, out_path, command):
    """Per-launch HBM traffic of the attention kernel from the two counter
    runs of `--traffic-job`: each counter (KiB per dispatch) is scaled by
    COPY_BYTES / (what it reads for the final copy dispatch)."""
    res = {}
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _counter_rows(d, counter)
        attn = [(i, v) for i, v in rows.items() if "attn_fp8_kernel" in v[0]]
        if len(attn) != 1:
            raise SystemExit(f"expected one attention dispatch in {d}, found {len(attn)}")
        copy_id = max(rows)
        copy_name, copy_kib = rows[copy_id]
        attn_kib = attn[0][1][1]
        factor = COPY_BYTES / (copy_kib * 1024.0)
        res[key] = {"counter": counter, "attn_kib": attn_kib, "copy_kib": copy_kib, "copy_kernel": copy_name[:80],
                    "factor": factor, "bytes": attn_kib * 1024.0 * factor}
    rec = {
        "kernel": "attn_fp8_kernel<128,true>",
        "workload": "wan: B=1 H=40 S=75600 D=128, V-Smooth",
        "kernel_source_sha256": _sha(ATTN_SRC),
        "fetch_bytes": res["fetch"]["bytes"],
        "write_bytes": res["write"]["bytes"],
        "bytes_per_launch": res["fetch"]["bytes"] + res["write"]["bytes"],
        "calibration": f"{COPY_BYTES}-byte device copy, last dispatch of the job",
        "counters": res,
        "command": command,
    }
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def prep_job(w):
    """The preparation passes once each on the workload: vc_quantize of Q, K
    and V, a cold vc_smooth_group (k-means from the Forgy draw), a
    vc_smooth_group reusing its permutation, then one plain device copy of
    COPY_BYTES as the very last dispatch (the FETCH_SIZE / WRITE_SIZE
    calibration of --counter-summary)."""
    import torch

    import bit_fp8_attention_amd as vc
    import vcsynth
    q, k, v = vcsynth.make_qkv(w.name, device="cuda")
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    vc.vc_quantize(q, k, v, sm_scale=w.sm_scale)
    g = vc.vc_smooth_group(k, v, w.clusters or 64, w.iters or 4, w.seed)
    vc.vc_smooth_group(k, v, w.clusters or 64, w.iters or 4, w.seed, reuse_perm=g["perm"])
    b.copy_(a)
    torch.cuda.synchronize()
    log("prep job done")


def attn4_job(w):
    """The 4-bit path once on the workload: the grouping it reuses (pi and
    the block means), vc_quantize4, one V-Smooth vc_attn_fwd4 launch, then
    one plain device copy of COPY_BYTES as the very last dispatch (the
    FETCH_SIZE / WRITE_SIZE calibration of --counter-summary)."""
    import torch

    import bit_fp8_attention_amd as vc
    import vcsynth
    q, k, v = vcsynth.make_qkv(w.name, device="cuda")
    g = vc.vc_smooth_group(k, v, w.clusters or 64, w.iters or 4, w.seed)
    z = vc.vc_quantize4(q, k, v, sm_scale=w.sm_scale, perm=g["perm"], mu_bf16=g["mu_bf16"])
    o = torch.empty_like(q)
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    vc.vc_attn_fwd4(z["q4"], z["q4_scale"], z["k4"], z["k4_scale"], z["v4"], z["v4_scale"], g["mu_bf16"], S=w.S,
                    out=o)
    b.copy_(a)
    torch.cuda.synchronize()
    log("attn4 job done")


def counter_summary(out_path, title, dirs, command):
    """Per-kernel table of every counter found under the rocprofv3 --pmc
    output directories: value per dispatch (averaged over the kernel's
    dispatches).  FETCH_SIZE and WRITE_SIZE (KiB per dispatch) also appear
    as bytes, scaled by COPY_BYTES / (the counter's reading for the last
    dispatch of the run, the calibration copy)."""
    import csv
    import glob
    per = {}    # kernel -> counter -> [values]
    calib = {}  # counter -> factor
    traces = [d[len("trace="):] for d in dirs if d.startswith("trace=")]
    dirs = [d for d in dirs if not d.startswith("trace=")]
    for d in dirs:
        by_disp = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    key = (int(r["Dispatch_Id"]), r["Counter_Name"])
                    name = r["Kernel_Name"]
                    prev = by_disp.get(key, (name, 0.0))
                    by_disp[key] = (name, prev[1] + float(r["Counter_Value"]))
        if not by_disp:
            raise SystemExit(f"no counter rows under {d}")
        last = max(k[0] for k in by_disp)
        for (did, ctr), (name, val) in by_disp.items():
            if did == last and ctr in ("FETCH_SIZE", "WRITE_SIZE"):
                calib[ctr] = COPY_BYTES / (val * 1024.0)
                continue
            if did == last or "vc::" not in name:  # the library's kernels only
                continue
            short = name.replace("vc::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
            per.setdefault(short, {}).setdefault(ctr, []).append(val)
    ctrs = sorted({c for v in per.values() for c in v})
    lines = [f"# {title}", "", "Command (from the repository root copied to the GPU host; OUT = gpurun_out):", "",
             "    " + command.replace("\n", "\n    "), "",
             "Library kernels only.  Value per dispatch, averaged over the kernel's dispatches; calls = dispatches "
             "seen."]
    if calib:
        lines.append("FETCH_SIZE / WRITE_SIZE as bytes: each KiB counter times " +
                     ", ".join(f"{c} {f:.3f}" for c, f in sorted(calib.items())) +
                     f" (the {COPY_BYTES}-byte calibration copy, last dispatch).")
    lines += ["", "| kernel | calls | " + " | ".join(ctrs) + " |", "|---|---|" + "---|" * len(ctrs)]
    for kname in sorted(per):
        row = per[kname]
        n = max(len(v) for v in row.values())
        cells = []
        for c in ctrs:
            if c not in row:
                cells.append("")
                continue
            m = sum(row[c]) / len(row[c])
            if c in calib:
                cells.append(f"{m * 1024.0 * calib[c] / 1e9:.4f} GB")
            else:
                cells.append(f"{m:.4g}")
        lines.append(f"| `{kname}` | {n} | " + " | ".join(cells) + " |")
    for d in traces:  # kernel-trace runs (--kernel-trace --stats): durations
        for f in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
            lines += ["", "Kernel durations (--kernel-trace --stats of the same job), microseconds:", "",
                      "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if "vc::" not in r["Name"]:
                        continue
                    short = r["Name"].replace("vc::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
                    lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                                 f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_baseline(w, q, k, v, target_s=12.0):
    """The oracle as it stands on head 0 of the same inputs: quantise and
    group the head (untimed, like the GPU's preparation), then emulate a
    growing number of full-length query rows until about target_s seconds."""
    import numpy as np

    import oracle
    import vcsynth
    qb = vcsynth.bf16_bits(q[:, :, :1])
    kb = vcsynth.bf16_bits(k[:, :, :1])
    vb = vcsynth.bf16_bits(v[:, :, :1])
    t0 = time.perf_counter()
    prep = oracle.pipeline_head(qb, kb, vb, 0, 0, vsmooth=w.vsmooth, nclust=w.clusters or 64, iters=w.iters or 4,
                                seed=w.seed, sm_scale=w.sm_scale, rows=np.array([0]))
    t_prep = time.perf_counter() - t0
    mu = prep.get("mu_scaled")
    kc = prep["k_codes"]
    ks = prep["k_scale"]
    vc_ = prep["r_codes"] if w.vsmooth else prep["v_codes"]
    vs = prep["r_scale"] if w.vsmooth else prep["v_scale"]
    rng = np.random.default_rng(0)
    n, elapsed = 8, 0.0
    while True:
        rows = np.sort(rng.choice(w.S, n, replace=False))
        t0 = time.perf_counter()
        oracle.attn_emulate_rows(prep["q_codes"], prep["q_scale"], kc, ks, vc_, vs, mu, w.S, 0.125, rows)
        elapsed = time.perf_counter() - t0
        if elapsed >= 0.8 * target_s or n >= w.S:
            break
        n = min(w.S, int(n * max(2.0, target_s / max(elapsed, 1e-3))))
    flops = 4.0 * n * w.S * w.D
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{n} query rows of head 0 (full {w.S}-key range, {'V-Smooth' if w.vsmooth else 'plain'} "
                   f"emulation) in {elapsed:.2f} s; the head's oracle quantise+grouping took {t_prep:.1f} s "
                   f"untimed; extrapolated full call {elapsed * w.S * w.H / n:.0f} s"),
    }


FP4_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4 matrix-core peak
HBM_PEAK_GBPS = 8000.0
ROUNDS = 31                # launches per leg in the interleaved sampling (median of these)
SETTLE_S = 2.0             # seconds of whole steps before anything is timed


class ClockSampler:
    """The GPU's shader clock (pp_dpm_sclk, the level marked '*') and board
    power (hwmon power1_input, else power1_average) sampled every few
    milliseconds on a host thread while a leg runs; each sample is tagged
    with the leg that was running when it was taken."""

    def __init__(self, torch, period=0.004):
        import glob
        import threading
        p = torch.cuda.get_device_properties(0)
        bus = "%04x:%02x:%02x" % (getattr(p, "pci_domain_id", 0), getattr(p, "pci_bus_id", 0),
                                  getattr(p, "pci_device_id", 0))
        self.sclk = (glob.glob(f"/sys/bus/pci/devices/{bus}*/pp_dpm_sclk") or [None])[0]
        pw = [c for c in glob.glob(f"/sys/bus/pci/devices/{bus}*/hwmon/hwmon*/power1_*")
              if c.endswith(("power1_input", "power1_average"))]
        self.power = sorted(pw, key=lambda c: not c.endswith("input"))[0] if pw else None
        self.period = period
        self.tag = None
        self.samples = []  # (tag, MHz or None, W or None)
        self._stop = False
        self._th = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        mhz = watts = None
        if self.sclk:
            try:
                for line in open(self.sclk).read().splitlines():
                    if line.rstrip().endswith("*"):
                        mhz = float(line.split(":")[1].strip().lower().split("mhz")[0])
            except (OSError, ValueError, IndexError):
                pass
        if self.power:
            try:
                watts = int(open(self.power).read()) / 1e6
            except (OSError, ValueError):
                pass
        return mhz, watts

    def _run(self):
        while not self._stop:
            tag = self.tag
            if tag is not None:
                mhz, watts = self._read()
                if tag == self.tag:  # still the same leg
                    self.samples.append((tag, mhz, watts))
            time.sleep(self.period)

    def __enter__(self):
        if self.sclk or self.power:
            self._th.start()
        return self

    def __exit__(self, *exc):
        self._stop = True
        if self._th.is_alive():
            self._th.join()

    def summary(self, tag):
        mhz = sorted(m for t, m, _ in self.samples if t == tag and m is not None)
        watts = [x for t, _, x in self.samples if t == tag and x is not None]
        if not mhz and not watts:
            return None
        return {"sclk_mhz_median": mhz[len(mhz) // 2] if mhz else None,
                "sclk_mhz_min": mhz[0] if mhz else None, "sclk_mhz_max": mhz[-1] if mhz else None,
                "board_power_w_mean": round(sum(watts) / len(watts), 1) if watts else None,
                "samples": max(len(mhz), len(watts))}


SPIN_MS = 0.5  # GPU spin ahead of each timed launch


def spin_cycles(ms_target):
    """Argument of torch.cuda._sleep that keeps the GPU busy for about
    ms_target (measured once with events)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    e0.record()
    torch.cuda._sleep(1_000_000)
    e1.record()
    e1.synchronize()
    return max(1000, int(1_000_000 * ms_target / max(e0.elapsed_time(e1), 1e-3)))


def interleaved(legs, rounds, seed, sampler):
    """Every leg once per round, in a freshly shuffled order each round (a
    seeded generator); each launch bracketed by HIP events on the stream it
    runs on and synchronised before the next, so it runs alone on the GPU.
    A short GPU spin is enqueued ahead of the start event, so that a call
    made of several kernel launches is fully queued when its bracket opens
    (its host-side enqueue time is not counted).  Two untimed launches of
    each leg first.  Returns name -> list of ms."""
    import random

    import torch
    names = list(legs)
    for name in names:
        for _ in range(2):
            legs[name]()
        torch.cuda.synchronize()
    spin = spin_cycles(SPIN_MS)
    rng = random.Random(seed)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms = {name: [] for name in names}
    for r in range(rounds):
        order = names[:]
        rng.shuffle(order)
        for name in order:
            sampler.tag = name
            torch.cuda._sleep(spin)
            e0.record()
            legs[name]()
            e1.record()
            e1.synchronize()
            sampler.tag = None
            ms[name].append(e0.elapsed_time(e1))
        if (r + 1) % 10 == 0 or r + 1 == rounds:
            log(f"interleaved round {r + 1}/{rounds} done")
    return ms


def _stat(xs):
    ys = sorted(xs)
    n = len(ys)
    med = ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])
    return {"median_ms": round(med, 4), "mean_ms": round(sum(ys) / n, 4), "min_ms": round(ys[0], 4),
            "max_ms": round(ys[-1], 4), "n": n}


def group_bytes(w, iters):
    """Algorithmic HBM bytes of a cold vc_smooth_group call and of a
    permutation-reuse call: iters k-means reads of V, the K/V gather, the
    second V' gather of the residual pass, the K' and R writes, labels and
    pi, the block means."""
    B, H, S, D = w.B, w.H, w.S, w.D
    nb = (S + 127) // 128
    bf = 2 * B * S * H * D            # one bf16 tensor
    f8 = B * H * nb * 128 * D         # one FP8 operand
    apply_b = 3 * bf + 2 * f8 + 8 * B * H * S + 6 * B * H * nb * D
    return iters * bf + apply_b, apply_b


def quantize_bytes(w, with_kv):
    """vc_quantize: read Q (and K, V) in bf16, write the FP8 codes and the
    per-block (per-head for V) scales."""
    B, H, S, D = w.B, w.H, w.S, w.D
    nb = (S + 127) // 128
    bf = 2 * B * S * H * D
    f8 = B * H * nb * 128 * D
    one = bf + f8 + 4 * B * H * nb
    return one * 3 if with_kv else one


def amortised(tg, tr, attn_ms, steps=50):
    """Grouping cost per step over a `steps`-step schedule ([VC] §3.4, App. A:
    grouping during the first ceil(steps / 4) steps, the permutation computed
    afresh every 4th of them and reused in between)."""
    window = -(-steps // 4)
    regroups = sum(1 for s in range(window) if s % 4 == 0)
    per_step = (regroups * tg + (window - regroups) * tr) / steps
    return {"steps": steps, "group_steps": window, "regroups": regroups, "ms_per_step": round(per_step, 4),
            "pct_of_attention": round(100 * per_step / attn_ms, 2)}


def _gbps(nbytes, ms):
    g = nbytes / (ms * 1e-3) / 1e9
    return {"gb": round(nbytes / 1e9, 3), "ms": round(ms, 4), "GBps": round(g, 1),
            "frac_hbm": round(g / HBM_PEAK_GBPS, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="wan")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-repair", action="store_true", help="skip the Open-VC repair-row measurement")
    ap.add_argument("--no-mxfp4", action="store_true", help="skip the 4-bit (MXFP4) path measurement")
    ap.add_argument("--no-m-leg", action="store_true", help="skip the H=48, S=84672 grouping legs")
    ap.add_argument("--rounds", type=int, default=ROUNDS, help="interleaved launches per leg (median)")
    ap.add_argument("--traffic-job", action="store_true",
                    help="one attention launch + calibration copy, for rocprofv3 --pmc runs")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "OUT_JSON", "COMMAND"),
                    help="write the per-launch traffic record from the two counter runs")
    ap.add_argument("--attn4-job", action="store_true",
                    help="one 4-bit V-Smooth launch, then a 1 GiB device copy (for rocprofv3 --pmc runs)")
    ap.add_argument("--prep-job", action="store_true",
                    help="the preparation passes once + calibration copy, for rocprofv3 --pmc runs")
    ap.add_argument("--counter-summary", nargs="+", metavar="ARG",
                    help="OUT_MD TITLE COMMAND DIR [DIR ...]: per-kernel counter table of --pmc runs "
                         "(a DIR given as trace=DIR is a --kernel-trace --stats run: durations)")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.counter_summary:
        a = args.counter_summary
        if len(a) < 4:
            raise SystemExit("--counter-summary OUT_MD TITLE COMMAND DIR [DIR ...]")
        counter_summary(a[0], a[1], a[3:], a[2])
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_fp8_attention_amd as vc
    import vcsynth

    w = vcsynth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.traffic_job:
        traffic_job(w)
        return
    if args.attn4_job:
        attn4_job(w)
        return
    if args.prep_job:
        prep_job(w)
        return
    t0 = time.perf_counter()
    q, k, v = vcsynth.make_qkv(w.name, device=dev)
    torch.cuda.synchronize()
    log(f"inputs {w.name} B={w.B} H={w.H} S={w.S} D={w.D} generated in {time.perf_counter() - t0:.1f} s")

    vs_on = w.vsmooth
    clusters, iters = (w.clusters, w.iters) if vs_on else (0, 0)
    qz = vc.vc_quantize(q, sm_scale=w.sm_scale) if vs_on else vc.vc_quantize(q, k, v, sm_scale=w.sm_scale)
    if vs_on:
        ws = torch.empty(vc.vc_smooth_group_workspace_size(w.B, w.H, w.S, w.D, clusters), dtype=torch.uint8,
                         device=dev)
        g = vc.vc_smooth_group(k, v, clusters, iters, w.seed, workspace=ws)
    o = torch.empty_like(q)
    torch.cuda.synchronize()

    def step(ev=None):
        E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        e = [E() for _ in range(4)] if ev is not None else None
        if e: e[0].record()
        if vs_on:
            vc.vc_quantize(q, sm_scale=w.sm_scale, out=qz)
            if e: e[1].record()
            vc.vc_smooth_group(k, v, clusters, iters, w.seed, workspace=ws, out=g)
            if e: e[2].record()
            vc.vc_attn_fwd(qz["q8"], qz["q_scale"], g["k8"], g["k_scale"], g["r8"], g["r_scale"], g["mu_split"],
                           S=w.S, out=o)
        else:
            vc.vc_quantize(q, k, v, sm_scale=w.sm_scale, out=qz)
            if e: e[1].record()
            if e: e[2].record()
            vc.vc_attn_fwd(qz["q8"], qz["q_scale"], qz["k8"], qz["k_scale"], qz["v8"], qz["v_scale"], None, S=w.S,
                           out=o)
        if e:
            e[3].record()
            ev.append(e)

    # ---- the clock and board power settle under load: the whole step,
    # repeated for at least 2 s, before anything is timed
    t_s, n_s = time.perf_counter(), 0
    while time.perf_counter() - t_s < SETTLE_S:
        step()
        torch.cuda.synchronize()
        n_s += 1
    log(f"settle: {n_s} steps in {time.perf_counter() - t_s:.1f} s")

    # ---- the step contract: W untimed steps, then exactly K whole-path steps
    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")
    evs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {wall:.3f} s")
    ms_per_step = wall * 1e3 / args.steps
    step_ms = {"vc_quantize": _stat([e[0].elapsed_time(e[1]) for e in evs]),
               "vc_smooth_group": _stat([e[1].elapsed_time(e[2]) for e in evs]),
               "vc_attn_fwd": _stat([e[2].elapsed_time(e[3]) for e in evs])}
    assert torch.isfinite(o.float()).all().item(), "non-finite attention output"

    # ---- the legs, sampled interleaved in random order -----------------------
    head = "fp8_vsmooth" if vs_on else "fp8_plain"
    legs = {}
    if vs_on:
        gr = {kk: vv for kk, vv in g.items() if kk not in ("centroids", "labels")}
        perm0 = g["perm"].clone()
        legs["fp8_vsmooth"] = lambda: vc.vc_attn_fwd(qz["q8"], qz["q_scale"], g["k8"], g["k_scale"], g["r8"],
                                                     g["r_scale"], g["mu_split"], S=w.S, out=o)
        legs["quantize_q"] = lambda: vc.vc_quantize(q, sm_scale=w.sm_scale, out=qz)
        legs["group"] = lambda: vc.vc_smooth_group(k, v, clusters, iters, w.seed, workspace=ws, out=g)
        legs["group_reuse"] = lambda: vc.vc_smooth_group(k, v, clusters, iters, w.seed, workspace=ws, out=gr,
                                                         reuse_perm=perm0)
    qp = qz if not vs_on else vc.vc_quantize(q, k, v, sm_scale=w.sm_scale)
    op = torch.empty_like(q)
    legs["fp8_plain"] = lambda: vc.vc_attn_fwd(qp["q8"], qp["q_scale"], qp["k8"], qp["k_scale"], qp["v8"],
                                               qp["v_scale"], None, S=w.S, out=op)
    legs["quantize_qkv"] = lambda: vc.vc_quantize(q, k, v, sm_scale=w.sm_scale, out=qp)
    if not args.no_bf16:
        vt = vc.vc_pack_v_bf16(v)
        ob = torch.empty_like(q)
        legs["bf16"] = lambda: vc.vc_attn_fwd_bf16(q, k, vt, out=ob, sm_scale=w.sm_scale)
    rho = 0.005
    if not args.no_repair:
        R = vc.repair_count(w.S, rho)
        rws = torch.empty(vc.vc_repair_workspace_size(w.B, w.H, w.S, w.D), dtype=torch.uint8, device=dev)
        rp = vc.vc_repair_prepare(k, v, R, workspace=rws)
        orp = torch.empty_like(q)
        legs["repair_prepare"] = lambda: vc.vc_repair_prepare(k, v, R, workspace=rws, out=rp)
        legs["fp8_plain_repair"] = lambda: vc.vc_attn_fwd(qp["q8"], qp["q_scale"], qp["k8"], qp["k_scale"],
                                                          qp["v8"], qp["v_scale"], None, S=w.S, out=orp, repair=rp)
    if not args.no_mxfp4 and vs_on:
        z4 = vc.vc_quantize4(q, k, v, sm_scale=w.sm_scale, perm=g["perm"], mu_bf16=g["mu_bf16"])
        o4 = torch.empty_like(q)
        legs["quantize4"] = lambda: vc.vc_quantize4(q, k, v, sm_scale=w.sm_scale, perm=perm0, mu_bf16=g["mu_bf16"],
                                                    out=z4)
        legs["attn4"] = lambda: vc.vc_attn_fwd4(z4["q4"], z4["q4_scale"], z4["k4"], z4["k4_scale"], z4["v4"],
                                                z4["v4_scale"], g["mu_bf16"], S=w.S, out=o4)
    # the larger video shape's grouping (its own tensors), with its attention
    # for the amortised share
    wm = vcsynth.WORKLOADS["minimax"]
    m_leg = vs_on and not args.no_m_leg and w.name != wm.name
    if m_leg:
        qm, km, vm = vcsynth.make_qkv(wm.name, device=dev)
        wsm = torch.empty(vc.vc_smooth_group_workspace_size(wm.B, wm.H, wm.S, wm.D, wm.clusters), dtype=torch.uint8,
                          device=dev)
        gm = vc.vc_smooth_group(km, vm, wm.clusters, wm.iters, wm.seed, workspace=wsm)
        grm = {kk: vv for kk, vv in gm.items() if kk not in ("centroids", "labels")}
        permm = gm["perm"].clone()
        qzm = vc.vc_quantize(qm, sm_scale=wm.sm_scale)
        om = torch.empty_like(qm)
        legs["M_group"] = lambda: vc.vc_smooth_group(km, vm, wm.clusters, wm.iters, wm.seed, workspace=wsm, out=gm)
        legs["M_group_reuse"] = lambda: vc.vc_smooth_group(km, vm, wm.clusters, wm.iters, wm.seed, workspace=wsm,
                                                           out=grm, reuse_perm=permm)
        legs["M_fp8_vsmooth"] = lambda: vc.vc_attn_fwd(qzm["q8"], qzm["q_scale"], gm["k8"], gm["k_scale"], gm["r8"],
                                                       gm["r_scale"], gm["mu_split"], S=wm.S, out=om)
    torch.cuda.synchronize()
    rounds = args.rounds
    t0 = time.perf_counter()
    with ClockSampler(torch) as clk:
        ms = interleaved(legs, rounds, seed=20260, sampler=clk)
    log(f"interleaved sampling: {len(legs)} legs x {rounds} rounds in {time.perf_counter() - t0:.1f} s")
    st = {name: _stat(x) for name, x in ms.items()}
    med = {name: x["median_ms"] for name, x in st.items()}
    outs = [o, op] + ([om] if m_leg else [])
    assert all(torch.isfinite(x.float()).all().item() for x in outs), "non-finite attention output"
    flops = w.flops()
    attn_ms = med[head]
    value = flops / (attn_ms * 1e-3) / 1e12
    clock = {name: clk.summary(name) for name in legs if clk.summary(name)}
    clock_src = {"sclk": clk.sclk, "power": clk.power}

    traffic = traffic_from_profile() if (w.name == "wan" and vs_on) else None
    roof = {"bound": "mfma", "achieved": round(value, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(value / FP8_PEAK_TFLOPS, 4), "traffic": traffic,
            "kernel": "attn_fp8_kernel<128,%s>" % ("true" if vs_on else "false"),
            "launch_ms_median": attn_ms, "launch_ms_mean": st[head]["mean_ms"], "launches": st[head]["n"],
            "flops_per_launch": flops}
    if clock.get(head, {}) and clock[head].get("sclk_mhz_median"):
        f_obs = clock[head]["sclk_mhz_median"]
        roof["clock_mhz_observed"] = f_obs
        roof["frac_of_peak_at_observed_clock"] = round(value / (FP8_PEAK_TFLOPS * f_obs / 2400.0), 4)

    bf16 = None
    if "bf16" in med:
        bt = flops / (med["bf16"] * 1e-3) / 1e12
        bf16 = {"ms": med["bf16"], "tflops": round(bt, 1), "frac_of_bf16_peak": round(bt / BF16_PEAK_TFLOPS, 4),
                "speedup_fp8_over_bf16": round(med["bf16"] / attn_ms, 3)}

    prep = None
    if vs_on:
        gb_cold, gb_reuse = group_bytes(w, iters)
        prep = {"vc_quantize_q": _gbps(quantize_bytes(w, False), med["quantize_q"]),
                "vc_quantize_qkv": _gbps(quantize_bytes(w, True), med["quantize_qkv"]),
                "vc_smooth_group": _gbps(gb_cold, med["group"]),
                "vc_smooth_group_reuse_perm": _gbps(gb_reuse, med["group_reuse"]),
                "grouping_amortised_50_steps": amortised(med["group"], med["group_reuse"], attn_ms)}
        if m_leg:
            gm_cold, gm_reuse = group_bytes(wm, wm.iters)
            prep["M"] = {"workload": f"{wm.name}: B={wm.B} H={wm.H} S={wm.S} D={wm.D}",
                         "vc_smooth_group": _gbps(gm_cold, med["M_group"]),
                         "vc_smooth_group_reuse_perm": _gbps(gm_reuse, med["M_group_reuse"]),
                         "attn_fp8_vsmooth_ms": med["M_fp8_vsmooth"],
                         "attn_tflops": round(wm.flops() / (med["M_fp8_vsmooth"] * 1e-3) / 1e12, 1),
                         "grouping_amortised_50_steps": amortised(med["M_group"], med["M_group_reuse"],
                                                                  med["M_fp8_vsmooth"])}
        log(f"prep: {prep}")

    repair = None
    if "fp8_plain_repair" in med:
        repair = {"rho": rho, "rows_per_head": R, "prepare_ms": med["repair_prepare"],
                  "attn_plain_ms": med["fp8_plain"], "attn_with_repair_ms": med["fp8_plain_repair"],
                  "overhead_pct": round(100 * (med["fp8_plain_repair"] / med["fp8_plain"] - 1), 2),
                  "tflops_with_repair": round(flops / (med["fp8_plain_repair"] * 1e-3) / 1e12, 1)}
        log(f"repair rows: {repair}")

    mx4 = None
    if "attn4" in med:
        tf = flops / (med["attn4"] * 1e-3) / 1e12
        mx4 = {"format": "MXFP4 (E2M1, E8M0 per 32)", "vsmooth": True, "quantize4_ms": med["quantize4"],
               "attn_ms": med["attn4"], "tflops": round(tf, 1), "frac_fp4_peak": round(tf / FP4_PEAK_TFLOPS, 4)}
        if "bf16" in med:  # the comparison the pages make for their 4-bit path
            mx4["speedup_over_bf16"] = round(med["bf16"] / med["attn4"], 3)
        log(f"mxfp4 path: {mx4}")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(w, q.cpu(), k.cpu(), v.cpu())
        log(f"cpu baseline: {cpu['sample']}")

    res = {
        "metric": "vc_attn_fwd TFLOP/s + % FP8 MFMA peak at H=40,S=75600,D=128",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} S={w.S} D={w.D}" +
                   (f" grid={'x'.join(map(str, w.grid))}" if w.grid else ""),
                   "vsmooth": vs_on, "clusters": clusters, "kmeans_iters": iters, "window": 2,
                   "sm_scale": w.sm_scale},
        "pct_fp8_peak": round(100 * value / FP8_PEAK_TFLOPS, 2),
        "timing": {"protocol": (f"{rounds} rounds; every round runs each leg once in a freshly shuffled order "
                                "(seeded); each launch bracketed by HIP events on its stream and synchronised "
                                f"before the next, behind a {SPIN_MS} ms GPU spin so that its kernels are all "
                                "queued when the bracket opens; value and every leg figure are medians"),
                   "legs": st},
        "clock": {"per_leg": clock, "source": clock_src},
        "step_breakdown_ms": step_ms,
        "path_tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "roofline": roof,
        "bf16_baseline": bf16,
        "prep_passes": prep,
        "open_vc_repair": repair,
        "mxfp4_path": mx4,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
