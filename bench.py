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


def repair_measurement(vc, w, q, k, v, flops, rho=0.005, n=3):
    """Open-VC's V residual repair on the same inputs, plain path: time of
    vc_repair_prepare for R = ceil(rho S) rows per head, and of vc_attn_fwd
    without and with the repair tiles (HIP events, mean of n launches)."""
    import torch

    qz = vc.vc_quantize(q, k, v, sm_scale=w.sm_scale)
    R = vc.repair_count(w.S, rho)
    ws = torch.empty(vc.vc_repair_workspace_size(w.B, w.H, w.S, w.D), dtype=torch.uint8, device=q.device)
    rp = vc.vc_repair_prepare(k, v, R, workspace=ws)
    o = torch.empty_like(q)
    args = (qz["q8"], qz["q_scale"], qz["k8"], qz["k_scale"], qz["v8"], qz["v_scale"], None)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / n

    t_prep = timed(lambda: vc.vc_repair_prepare(k, v, R, workspace=ws, out=rp))
    t_plain = timed(lambda: vc.vc_attn_fwd(*args, S=w.S, out=o))
    t_rep = timed(lambda: vc.vc_attn_fwd(*args, S=w.S, out=o, repair=rp))
    del qz, rp, ws, o
    return {"rho": rho, "rows_per_head": R, "prepare_ms": round(t_prep, 3), "attn_plain_ms": round(t_plain, 3),
            "attn_with_repair_ms": round(t_rep, 3),
            "tflops_with_repair": round(flops / (t_rep * 1e-3) / 1e12, 1)}


FP4_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4 matrix-core peak
HBM_PEAK_GBPS = 8000.0


def prep_measurement(vc, w, q, k, v, qz, g, ws, clusters, iters, attn_ms, ms_q, ms_g, n=3):
    """The preparation passes against HBM bandwidth (algorithmic bytes over
    their timed mean), and the grouping cost amortised over a 50-step
    schedule ([VC] §3.4 and App. A: grouping on the first ceil(50 / 4) = 13
    steps, the permutation recomputed at steps 0, 4, 8, 12 and reused in
    between), as a share of one attention call."""
    import torch

    B, H, S, D = w.B, w.H, w.S, w.D
    nb = (S + 127) // 128
    bf = 2 * B * S * H * D            # one bf16 tensor
    f8 = B * H * nb * 128 * D         # one FP8 operand
    q_bytes = bf + f8 + 4 * B * H * nb
    apply_bytes = 3 * bf + 2 * f8 + 8 * B * H * S + 6 * B * H * nb * D  # gather K, V; residual pass; K', R; labels, pi; means
    group_bytes = iters * bf + apply_bytes
    tq = sum(ms_q) / len(ms_q)
    tg = sum(ms_g) / len(ms_g)
    # the reuse step: the permutation of the last grouping, gather + means + residuals only
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    vc.vc_smooth_group(k, v, clusters, iters, w.seed, workspace=ws, out=dict(g), reuse_perm=g["perm"])
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        vc.vc_smooth_group(k, v, clusters, iters, w.seed, workspace=ws, out=dict(g), reuse_perm=g["perm"])
    e1.record()
    e1.synchronize()
    tr = e0.elapsed_time(e1) / n
    steps, window = 50, 13
    regroups = sum(1 for s in range(window) if s % 4 == 0)
    per_step = (regroups * tg + (window - regroups) * tr) / steps
    gb = lambda b, t: round(b / (t * 1e-3) / 1e9, 1)  # noqa: E731
    return {"vc_quantize_q": {"gb": round(q_bytes / 1e9, 3), "ms": round(tq, 3), "GBps": gb(q_bytes, tq),
                              "frac_hbm": round(gb(q_bytes, tq) / HBM_PEAK_GBPS, 3)},
            "vc_smooth_group": {"gb": round(group_bytes / 1e9, 3), "ms": round(tg, 3), "GBps": gb(group_bytes, tg),
                                "frac_hbm": round(gb(group_bytes, tg) / HBM_PEAK_GBPS, 3)},
            "vc_smooth_group_reuse_perm": {"gb": round(apply_bytes / 1e9, 3), "ms": round(tr, 3),
                                           "GBps": gb(apply_bytes, tr),
                                           "frac_hbm": round(gb(apply_bytes, tr) / HBM_PEAK_GBPS, 3)},
            "grouping_amortised_50_steps": {"ms_per_step": round(per_step, 3),
                                            "pct_of_attention": round(100 * per_step / attn_ms, 2)}}


def mxfp4_measurement(vc, w, q, k, v, g, flops, n=3):
    """The 4-bit path (V-Smooth without ExpCast, MXFP4) on the same inputs and
    grouping: vc_quantize4 (Q, and K/V through pi minus the block means) and
    vc_attn_fwd4, HIP events, mean of n launches after one warm-up."""
    import torch

    z = vc.vc_quantize4(q, k, v, sm_scale=w.sm_scale, perm=g["perm"], mu_bf16=g["mu_bf16"])
    o = torch.empty_like(q)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / n

    tq = timed(lambda: vc.vc_quantize4(q, k, v, sm_scale=w.sm_scale, perm=g["perm"], mu_bf16=g["mu_bf16"], out=z))
    ta = timed(lambda: vc.vc_attn_fwd4(z["q4"], z["q4_scale"], z["k4"], z["k4_scale"], z["v4"], z["v4_scale"],
                                       g["mu_bf16"], S=w.S, out=o))
    tf = flops / (ta * 1e-3) / 1e12
    del z, o
    return {"format": "MXFP4 (E2M1, E8M0 per 32)", "vsmooth": True, "quantize4_ms": round(tq, 3),
            "attn_ms": round(ta, 3), "tflops": round(tf, 1), "frac_fp4_peak": round(tf / FP4_PEAK_TFLOPS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="wan")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-repair", action="store_true", help="skip the Open-VC repair-row measurement")
    ap.add_argument("--no-mxfp4", action="store_true", help="skip the 4-bit (MXFP4) path measurement")
    ap.add_argument("--traffic-job", action="store_true",
                    help="one attention launch + calibration copy, for rocprofv3 --pmc runs")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "OUT_JSON", "COMMAND"),
                    help="write the per-launch traffic record from the two counter runs")
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
    ms_q = [e[0].elapsed_time(e[1]) for e in evs]
    ms_g = [e[1].elapsed_time(e[2]) for e in evs]
    ms_a = [e[2].elapsed_time(e[3]) for e in evs]
    flops = w.flops()
    attn_ms = sum(ms_a) / len(ms_a)
    value = flops / (attn_ms * 1e-3) / 1e12
    ms_per_step = wall * 1e3 / args.steps
    assert torch.isfinite(o.float()).all().item(), "non-finite attention output"

    traffic = traffic_from_profile() if (w.name == "wan" and vs_on) else None
    roof = {"bound": "mfma", "achieved": round(value, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(value / FP8_PEAK_TFLOPS, 4), "traffic": traffic,
            "kernel": "attn_fp8_kernel<128,%s>" % ("true" if vs_on else "false"),
            "avg_launch_ms": round(attn_ms, 4), "flops_per_launch": flops}

    bf16 = None
    if not args.no_bf16:
        try:
            vt = vc.vc_pack_v_bf16(v)
            ob = torch.empty_like(q)
            for _ in range(2):
                vc.vc_attn_fwd_bf16(q, k, vt, out=ob, sm_scale=w.sm_scale)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = max(3, args.steps)
            e0.record()
            for _ in range(n):
                vc.vc_attn_fwd_bf16(q, k, vt, out=ob, sm_scale=w.sm_scale)
            e1.record()
            e1.synchronize()
            bms = e0.elapsed_time(e1) / n
            bt = flops / (bms * 1e-3) / 1e12
            bf16 = {"ms": round(bms, 3), "tflops": round(bt, 1), "frac_of_bf16_peak": round(bt / BF16_PEAK_TFLOPS, 4),
                    "speedup_fp8_over_bf16": round(bms / attn_ms, 3)}
            del vt, ob
        except vc.VcError as ex:
            log(f"bf16 baseline unavailable: {ex}")

    prep = None
    if vs_on:
        prep = prep_measurement(vc, w, q, k, v, qz, g, ws, clusters, iters, attn_ms, ms_q, ms_g)
        log(f"prep: {prep}")

    repair = None
    if not args.no_repair:
        repair = repair_measurement(vc, w, q, k, v, flops)
        log(f"repair rows: {repair}")

    mx4 = None
    if not args.no_mxfp4 and vs_on:
        mx4 = mxfp4_measurement(vc, w, q, k, v, g, flops)
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
        "breakdown_ms": {"vc_quantize": round(sum(ms_q) / len(ms_q), 3),
                         "vc_smooth_group": round(sum(ms_g) / len(ms_g), 3),
                         "vc_attn_fwd": round(attn_ms, 3)},
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
