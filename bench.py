#!/usr/bin/env python3
"""Throughput of the fused attention JVP (O, dO, LSE, dLSE) on one MI355X.

One step is one attn_jvp_fwd call over the whole workload with the inputs
already resident in HBM.  The timed region is bracketed by device
synchronisation and timed with HIP events recorded on the stream the kernel
is launched on.  Counted FLOPs are 6 * (visible query-key pairs) * (d_qk +
d_v) per (batch, head): the six products of the definition (QK^T, dQ K^T,
Q dK^T over d_qk; P V, P dV, (P . dS) V over d_v), 12 N^2 d when square.

``--shape B,H,Lq,Lkv,d_qk,d_v`` times a synthetic shape instead of a named
workload (Gaussian inputs, tangents x 0.1; ``--dtype fp32`` for float32);
``--splitkv S`` times the split-KV path (attn_jvp_fwd_splitkv with S splits, 0 = the library's
choice; the workspace is allocated once, outside the timed region);
``--backward`` times the primal backward (attn_jvp_bwd, with the workload's
mask if it has one) instead, on O and LSE from one forward call and a
Gaussian dL/dO, counting the algorithmic 10 * (visible pairs) * d FLOPs per
(batch, head) (S, dP, dV, dK, dQ; the recomputation of S and dP in the
second launch is not counted).

The warm-up runs at least ``--warmup`` steps and at least 0.3 s of work, so
the timed steps run at the sustained engine clock (``warmup_run`` in the
JSON line is the number of warm-up steps actually run).

Prints one JSON line.  ``--gpus`` above 1 is refused: this path runs on one
GPU.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention-JVP TFLOP/s (fwd+tangent) and % of bf16 MFMA peak, 1 GPU"
# MI355X dense MFMA peaks, TFLOP/s
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}
WARM_SECONDS = 0.3   # minimum warm-up before the timed steps
NAMES = ("q", "k", "v", "dq", "dk", "dv")
KERNEL_SOURCES = os.path.join(ROOT, "attention_jvp_amd", "csrc")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def visible_pairs(N, mask):
    """Number of (query, key) pairs the frame-window mask leaves visible."""
    if mask is None:
        return N * N
    F, T, C = mask["frames"], mask["tokens_per_frame"], mask["chunk_frames"]
    R = mask["radius_chunks"]
    anchors = set()
    if mask.get("anchor_first", 1):
        anchors.add(0)
    if mask.get("anchor_last", 1):
        anchors.add(F - 1)
    total = 0
    for qf in range(F):
        if mask.get("anchor_queries_see_all", 0) and qf in anchors:
            total += F
            continue
        seen = {f for f in range(F) if abs(f // C - qf // C) <= R} | anchors
        total += len(seen)
    return total * T * T


def kernel_sha():
    """sha256 over the sources of the forward attention kernel itself: the
    template (kernel.h), its launch geometry (plan.h) and its instance units
    (inst.h, inst_bf16_*.hip, inst_fp32.hip), by name."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_SOURCES)):
        if name in ("kernel.h", "plan.h", "inst.h", "inst_fp32.hip") or \
                name.startswith("inst_bf16_"):
            h.update(name.encode())
            with open(os.path.join(KERNEL_SOURCES, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def traffic_record(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha256") != kernel_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(w, x, target_s, gpu_out=None):
    """Time the float64 oracle on a bounded row sample of the same workload,
    and (with gpu_out, the outputs of a timed launch) compare the GPU's rows
    of that sample with the oracle's: normwise error of O, dO, dLSE and the
    absolute error of LSE in nats."""
    import numpy as np
    from oracle import FrameWindow, attention_jvp_rows

    vis = None
    if x["mask"] is not None:
        m = x["mask"]
        vis = FrameWindow(m["frames"], m["tokens_per_frame"], m["chunk_frames"],
                          m["radius_chunks"], bool(m["anchor_first"]), bool(m["anchor_last"]),
                          bool(m["anchor_queries_see_all"]))
    arrs = [x[n].float().numpy() for n in NAMES]

    def run(nrows):
        rows = np.linspace(0, w.N - 1, nrows).astype(np.int64)
        t0 = time.perf_counter()
        ref = attention_jvp_rows(*arrs, rows, visible=vis)
        return time.perf_counter() - t0, rows, ref

    # calibrate t(n) = fixed + n * per_row from two short runs (the fixed
    # part is the per-head widening of K, V, dK, dV to float64)
    t16, _, _ = run(16)
    t64, _, _ = run(64)
    per_row = max((t64 - t16) / 48, 1e-9)
    fixed = max(t16 - 16 * per_row, 0.0)
    nrows = int(max(16, min(w.N, (target_s - fixed) / per_row)))
    dt, rows, ref = run(nrows)
    if vis is None:
        pairs = len(rows) * w.Nkv
    else:
        pairs = int(vis(rows, np.arange(w.Nkv)).sum())
    flops = 6.0 * w.B * w.H * pairs * (w.d + w.dv)
    parity = None
    if gpu_out is not None:
        import torch
        idx = torch.from_numpy(rows).to(gpu_out[0].device)
        got = [t.index_select(2, idx).double().cpu().numpy() for t in gpu_out]
        parity = {"rows_per_head": int(len(rows))}
        for name, g, r in zip(("O", "dO", "LSE", "dLSE"), got, ref):
            fin = np.isfinite(r)
            diff = float(np.max(np.abs(g[fin] - r[fin]))) if fin.any() else 0.0
            if name == "LSE":
                parity["LSE_abs_nats"] = diff
            else:
                den = float(np.max(np.abs(r[fin]))) if fin.any() else 1.0
                parity[name + "_normwise"] = diff / max(den, 1e-30)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": blas_threads(),
        "affinity_cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"{len(rows)} evenly spaced query rows x {w.B * w.H} heads of {w.name} "
                   f"against all {w.Nkv} keys, float64 numpy; {dt:.1f} s"),
    }, parity


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="image_dit_4096")
    ap.add_argument("--shape", default=None, metavar="B,H,Lq,Lkv,DQK,DV",
                    help="time this synthetic shape instead of a named workload")
    ap.add_argument("--dtype", default="bf16", choices=("bf16", "fp32"),
                    help="element type of a --shape workload")
    ap.add_argument("--splitkv", type=int, default=-1, metavar="S",
                    help="time attn_jvp_fwd_splitkv with S key splits (0 = library choice)")
    ap.add_argument("--flush", action="store_true",
                    help="also time launches after writing 512 MiB (evicts L2 and MALL)")
    ap.add_argument("--backward", action="store_true",
                    help="time the primal backward (attn_jvp_bwd) instead of the JVP")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target length of the timed oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of the benchmark, run --steps plain device copies of "
                         "BYTES bytes (a known-size reference for HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this attention-JVP path has no "
              "multi-GPU form here (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, device="cuda", dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "copies": args.steps}), flush=True)
        return

    import attention_jvp_amd as aj
    from synth import WORKLOADS, Workload, make_inputs

    if args.shape:
        B, H, Lq, Lkv, dqk, dv = (int(t) for t in args.shape.split(","))
        w = Workload(f"shape_{B}x{H}x{Lq}x{Lkv}x{dqk}x{dv}", B, H, Lq, dqk, args.dtype, 1,
                     tangent_scale=0.1, n_kv=Lkv, d_v=dv)
    else:
        w = WORKLOADS[args.workload]
    log(f"workload {w.name}: B={w.B} H={w.H} Lq={w.N} Lkv={w.Nkv} d_qk={w.d} d_v={w.dv} {w.dtype}")
    x = make_inputs(w)
    g = [x[n].cuda() for n in NAMES]
    o = torch.empty((w.B, w.H, w.N, w.dv), device="cuda", dtype=g[0].dtype)
    do = torch.empty_like(o)
    lse = torch.empty((w.B, w.H, w.N), device="cuda", dtype=torch.float32)
    dlse = torch.empty_like(lse)
    outs = (o, do, lse, dlse)
    mask = x["mask"]
    splits = None
    if args.splitkv >= 0:
        dt = aj.ATTN_JVP_BF16 if w.dtype == "bf16" else aj.ATTN_JVP_FP32
        splits, need = aj.attn_jvp_splitkv_plan(aj.Shape(w.B, w.H, w.N, w.Nkv, w.d, w.dv), dt,
                                                mask, args.splitkv)
        ws = torch.empty(max(need, 256), device="cuda", dtype=torch.uint8)
        log(f"split-KV: {splits} splits, workspace {need} bytes")

    if args.backward:
        if splits is not None or w.dv != w.d:
            print("--backward: one head dim, no split-KV", file=sys.stderr)
            sys.exit(2)
        aj.fwd(*g, mask=mask, out=outs)
        go = torch.randn(o.shape, generator=torch.Generator().manual_seed(7)).to(o.dtype).cuda()
        grads = (torch.empty_like(g[0]), torch.empty_like(g[1]), torch.empty_like(g[2]),
                 torch.empty_like(lse))

    def step():
        if args.backward:
            aj.bwd(g[0], g[1], g[2], o, go, lse, mask=mask, out=grads)
        elif splits is None:
            aj.fwd(*g, mask=mask, out=outs)
        else:
            aj.fwd_splitkv(*g, mask=mask, num_splits=splits, workspace=ws, out=outs)

    # warm-up: W steps, continued until WARM_SECONDS of work have run, so
    # the timed steps see the sustained engine clock (a GPU coming out of idle
    # ramps its clock over the first tens of milliseconds of work)
    t_warm = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t_warm < WARM_SECONDS:
        step()
        n_warm += 1
        if n_warm % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps

    # per-launch times over a second run of the same number of steps (median,
    # minimum), and optionally with L2/MALL evicted before each launch
    def per_launch(before=None):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in evs:
            if before is not None:
                before()
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in evs)

    per = per_launch()
    timing = {"ms_mean": round(ms, 5), "ms_median": round(per[len(per) // 2], 5),
              "ms_min": round(per[0], 5)}
    if args.flush:
        junk = torch.empty(512 << 20, device="cuda", dtype=torch.uint8)
        cold = per_launch(lambda: junk.zero_())
        timing["ms_median_cold_l2_mall"] = round(cold[len(cold) // 2], 5)
        del junk
    pairs = visible_pairs(w.N, mask) if mask is not None else w.N * w.Nkv
    flops = 6.0 * w.B * w.H * pairs * (w.d + w.dv)
    if args.backward:
        flops = 10.0 * w.B * w.H * pairs * w.d
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    log(f"{ms:.4f} ms/step, {tflops:.1f} TFLOP/s ({100 * tflops / peak:.1f}% of {peak} peak)")

    cpu = parity = None
    if not args.no_cpu_baseline and not args.backward:
        log("timing the float64 oracle on a row sample (and checking the GPU's rows of it)")
        cpu, parity = cpu_baseline(w, x, args.cpu_seconds, gpu_out=outs)
        log(f"oracle: {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads; parity {parity}")

    line = {
        "metric": METRIC if not args.backward else
        "attention primal backward TFLOP/s (dQ, dK, dV) and % of bf16 MFMA peak, 1 GPU",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": n_warm,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "pct_of_peak": round(100 * tflops / peak, 2),
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "seed": w.seed,
            **({"Lkv": w.Nkv, "d_v": w.dv} if (w.Nkv != w.N or w.dv != w.d) else {}),
            **({"splitkv": splits} if splits is not None else {}),
            **({"pass": "backward"} if args.backward else {}),
            "mask": mask, "visible_pairs_per_head": pairs,
            "counted_flops": flops,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "traffic": traffic_record(w.name) if splits is None and not args.backward else None,
        },
        "cpu_baseline": cpu,
        "parity": parity,
        "timing": timing,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
