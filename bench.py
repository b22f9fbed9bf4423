"""Benchmark of the fused attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one fa_fwd call (the whole fused forward pass: scores, online
softmax, P.V, normalisation, lse) over the workload's seeded inputs, which are
resident in device memory before timing starts.  Prints one JSON line.  The
decode-shaped workloads (few queries, long keys) run one fa_fwd_split call per
step instead: the partial-result kernel over the key ranges and the merge,
with the workspace allocated before timing.  The gemm_* workloads time one
gemm_bias_gelu call per step (C = gelu(A W^T + bias)).

Reported alongside the throughput:
  * roofline: the attention kernel against the dense fp16/bf16 MFMA peak,
    with achieved = algorithmic FLOP per launch / mean launch time measured
    with HIP events on the launch stream over the timed region; traffic =
    HBM bytes per launch from rocprofv3 counters when they were taken on the
    current kernel source (else null);
  * cpu_baseline: the float64 oracle timed on this host's cores over a
    bounded sample of the same workload's rows;
  * a sampled parity check of the timed output against the oracle.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fa_inputs as fi  # noqa: E402

# MI355X dense MFMA peak for fp16/bf16: 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU.
PEAK_TFLOPS_F16 = 2516.6
# MI355X HBM3E peak bandwidth (8 TB/s).
PEAK_HBM_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "tile_level_programming_amd", "csrc", "fa_fwd.hip")
GEMM_SRC = os.path.join(ROOT, "tile_level_programming_amd", "csrc", "gemm_bias_gelu.hip")
ROWWISE_SRC = os.path.join(ROOT, "tile_level_programming_amd", "csrc", "rowwise.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash(path: str | None = None) -> str:
    """sha256[:16] of a kernel source (the attention one by default) with //
    comments and blank lines removed: counters taken on a source stay valid
    across comment edits, not code edits."""
    import re

    with open(path or KERNEL_SRC, encoding="utf-8") as f:
        lines = [re.sub(r"\s*//.*$", "", ln).rstrip() for ln in f]
    code = "\n".join(ln for ln in lines if ln)
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_for(workload: str, src: str | None = None):
    """HBM bytes per launch measured by rocprofv3 on this kernel source, or None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("kernel_sha256_16") != kernel_hash(src):
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(w, q, k, v, seconds: float, threads: int):
    import oracle

    per_row_flop = 4 * w.D * (w.unmasked_pairs() / w.Sq)  # algorithmic FLOP per query row, on average
    rng = np.random.default_rng(1234)
    total_rows = w.B * w.H * w.Sq
    # grow a calibration batch until it takes >= 1 s, then size the timed
    # sample to about `seconds` of work
    n = threads * 4
    while True:
        rows = rng.integers(0, total_rows, n)
        t0 = time.perf_counter()
        oracle.attention_rows(q, k, v, w.dtype, w.scale, w.causal, rows, threads=threads)
        dt = time.perf_counter() - t0
        if dt >= 1.0 or n >= total_rows:
            break
        n *= 4
    n = int(max(threads, min(total_rows, n * seconds / max(dt, 1e-6))))
    rows = rng.integers(0, total_rows, n)
    t0 = time.perf_counter()
    oracle.attention_rows(q, k, v, w.dtype, w.scale, w.causal, rows, threads=threads)
    dt = time.perf_counter() - t0
    return {
        "value": round(n * per_row_flop / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n} seeded random query rows of {w.name} ({n / total_rows:.2%} of the rows), "
                  f"float64, explicit scores over all {w.Sk} keys per row, {dt:.1f} s wall",
    }


def gemm_cpu_baseline(w, a, wt, b, seconds: float, threads: int):
    import oracle.gemm as og

    per_row_flop = 2 * w.N * w.K
    rng = np.random.default_rng(4321)
    n = threads
    while True:
        rows = rng.integers(0, w.M, n)
        t0 = time.perf_counter()
        og.gemm_rows(a, wt, b, w.dtype, rows=rows, threads=threads)
        dt = time.perf_counter() - t0
        if dt >= 1.0 or n >= w.M:
            break
        n *= 4
    n = int(max(threads, min(w.M, n * seconds / max(dt, 1e-6))))
    rows = rng.integers(0, w.M, n)
    t0 = time.perf_counter()
    og.gemm_rows(a, wt, b, w.dtype, rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    return {
        "value": round(n * per_row_flop / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n} seeded random output rows of {w.name} ({n / w.M:.2%} of the rows, all {w.N} columns each), "
                  f"float64, {dt:.1f} s wall",
    }


def run_gemm(args, w):
    """One step = one gemm_bias_gelu call: C = gelu(A W^T + bias)."""
    import torch

    from tile_level_programming_amd import fa

    log(f"[bench] workload {w.name}: generating seeded inputs")
    a, wt, b = fi.make_gemm_inputs(w)
    tdt = torch.float16 if w.dtype == "f16" else torch.bfloat16
    dev = torch.device("cuda:0")
    ad, wd = (torch.from_numpy(x.view(np.int16)).view(tdt).to(dev) for x in (a, wt))
    bd = torch.from_numpy(b.view(np.int16)).view(tdt).to(dev) if b is not None else None
    c = torch.empty((w.M, w.N), dtype=tdt, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    dt_code = fa.FA_F16 if w.dtype == "f16" else fa.FA_BF16

    def step():
        st = fa.gemm_bias_gelu(ad.data_ptr(), wd.data_ptr(), 0 if bd is None else bd.data_ptr(), c.data_ptr(),
                               w.M, w.N, w.K, dt_code, sp)
        if st != fa.FA_OK:
            raise fa.FaError(st)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    start.record(stream)
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    launch_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    ms_kernel = float(np.mean(launch_ms))
    flop = w.flops()
    tflops = flop / (ms * 1e-3) / 1e12
    tflops_kernel = flop / (ms_kernel * 1e-3) / 1e12
    log(f"[bench] {args.steps} steps: {ms:.4f} ms/step, {tflops:.1f} TFLOP/s; per launch mean {ms_kernel:.4f} ms "
        f"(min {min(launch_ms):.4f}, max {max(launch_ms):.4f}), {tflops_kernel:.1f} TFLOP/s")

    import oracle.gemm as og

    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, w.M - 1], rng.integers(0, w.M, 30)]))
    cs = c[torch.from_numpy(rows).to(dev)].double().cpu().numpy()
    threads = min(16, os.cpu_count() or 1)
    ref = og.gemm_rows(a, wt, b, w.dtype, rows=rows, threads=threads)
    rel = 2.0 ** -10 if w.dtype == "f16" else 2.0 ** -7
    err = float((np.abs(cs - ref) / np.maximum(np.abs(ref), 1.0)).max())
    parity_ok = bool(err <= rel and np.isfinite(cs).all())
    log(f"[bench] sampled parity: max |dC|/max(|C|,1) = {err:.2e} (bar {rel:.2e}) ok={parity_ok}")
    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {threads} threads, ~{args.cpu_seconds:.0f} s")
        cpu = gemm_cpu_baseline(w, a, wt, b, args.cpu_seconds, threads)
    line = {
        "metric": "GEMM + bias + GELU TFLOP/s and % of MI355X dense fp16/bf16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded i.i.d. normal A; W normal with sigma 1/sqrt(K); normal bias)",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "bias": w.bias, "algorithmic_flop": flop,
                   "algorithmic_bytes": w.io_bytes(), "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * tflops / PEAK_TFLOPS_F16, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops_kernel, 2), "peak": PEAK_TFLOPS_F16,
                     "unit": "TFLOP/s", "frac": round(tflops_kernel / PEAK_TFLOPS_F16, 4),
                     "traffic": traffic_for(w.name, GEMM_SRC), "kernel_ms": round(ms_kernel, 5),
                     "algorithmic_flop_per_launch": flop},
        "cpu_baseline": cpu,
        "parity_sample": {"rows": int(rows.size), "max_rel_err": err, "bar": rel, "ok": parity_ok},
        "kernel_sha256_16": kernel_hash(GEMM_SRC),
    }
    print(json.dumps(line), flush=True)


def run_rows(args, w):
    """One step = one row_softmax or rmsnorm_silu call over the workload's rows."""
    import torch

    import oracle.rowwise as orw
    from tile_level_programming_amd import fa

    log(f"[bench] workload {w.name}: generating seeded inputs")
    x, g = fi.make_row_inputs(w)
    tdt = torch.float16 if w.dtype == "f16" else torch.bfloat16
    dev = torch.device("cuda:0")
    xd = torch.from_numpy(x.view(np.int16)).view(tdt).to(dev)
    gd = torch.from_numpy(g.view(np.int16)).view(tdt).to(dev) if g is not None else None
    y = torch.empty_like(xd)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    dt_code = fa.FA_F16 if w.dtype == "f16" else fa.FA_BF16

    def step():
        if w.op == "softmax":
            st = fa.row_softmax(xd.data_ptr(), y.data_ptr(), w.R, w.C, dt_code, sp)
        else:
            st = fa.rmsnorm_silu(xd.data_ptr(), gd.data_ptr(), y.data_ptr(), w.R, w.C, w.eps, dt_code, sp)
        if st != fa.FA_OK:
            raise fa.FaError(st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    start.record(stream)
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    launch_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    ms_kernel = float(np.mean(launch_ms))
    nbytes = w.io_bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    gbs_kernel = nbytes / (ms_kernel * 1e-3) / 1e9
    log(f"[bench] {args.steps} steps: {ms:.4f} ms/step, {gbs:.0f} GB/s; per launch mean {ms_kernel:.4f} ms "
        f"(min {min(launch_ms):.4f}, max {max(launch_ms):.4f}), {gbs_kernel:.0f} GB/s")

    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, w.R - 1], rng.integers(0, w.R, 62)]))
    ys = y[torch.from_numpy(rows).to(dev)].double().cpu().numpy()
    threads = min(16, os.cpu_count() or 1)
    ref = (orw.softmax_rows(x, w.dtype, rows=rows, threads=threads) if w.op == "softmax"
           else orw.rmsnorm_silu_rows(x, g, w.dtype, w.eps, rows=rows, threads=threads))
    rel = 2.0 ** -10 if w.dtype == "f16" else 2.0 ** -7
    floor = (2.0 ** -24 if w.dtype == "f16" else 1e-30) if w.op == "softmax" else 1e-5
    over = float((np.abs(ys - ref) - (rel * np.abs(ref) + floor)).max())
    parity_ok = bool(over <= 0 and np.isfinite(ys).all())
    log(f"[bench] sampled parity: max (|dy| - bar) = {over:.2e} ok={parity_ok}")
    cpu = None
    if not args.no_cpu_baseline:
        n = min(w.R, max(threads, int(args.cpu_seconds * 2e8 / (w.C * 20))))
        rws = rng.integers(0, w.R, n)
        t0 = time.perf_counter()
        if w.op == "softmax":
            orw.softmax_rows(x, w.dtype, rows=rws, threads=threads)
        else:
            orw.rmsnorm_silu_rows(x, g, w.dtype, w.eps, rows=rws, threads=threads)
        dtc = time.perf_counter() - t0
        cpu = {"value": round(n * w.C * 4 / dtc / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"{n} seeded random rows of {w.name} ({n / w.R:.2%}), float64, {dtc:.2f} s wall"}
    line = {
        "metric": f"{w.op} GB/s of algorithmic bytes and % of MI355X HBM peak",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded i.i.d. normal rows" + (", normal weight)" if g is not None else ")"),
        "config": {"workload": w.name, "op": w.op, "R": w.R, "C": w.C, "algorithmic_bytes": nbytes,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs_kernel, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs_kernel / PEAK_HBM_GBS, 4), "traffic": traffic_for(w.name, ROWWISE_SRC),
                     "kernel_ms": round(ms_kernel, 5), "algorithmic_bytes_per_launch": nbytes},
        "cpu_baseline": cpu,
        "parity_sample": {"rows": int(rows.size), "max_excess_over_bar": over, "ok": parity_ok},
        "kernel_sha256_16": kernel_hash(ROWWISE_SRC),
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=fi.HEADLINE, choices=list(fi.ALL_WORKLOADS) + list(fi.GEMM_WORKLOADS)
                    + list(fi.ROW_WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB 10 times (calibrates the "
                         "HBM byte counters against a kernel of known traffic) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the attention path shards over (batch, head) with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from tile_level_programming_amd import fa

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: 10 copies of {n} bytes (read {n} B + write {n} B each)")
        return

    if args.workload in fi.GEMM_WORKLOADS:
        run_gemm(args, fi.GEMM_WORKLOADS[args.workload])
        return
    if args.workload in fi.ROW_WORKLOADS:
        run_rows(args, fi.ROW_WORKLOADS[args.workload])
        return
    w = fi.ALL_WORKLOADS[args.workload]
    log(f"[bench] workload {w.name}: generating seeded inputs")
    q, k, v = fi.make_inputs(w)
    tdt = torch.float16 if w.dtype == "f16" else torch.bfloat16
    dev = torch.device("cuda:0")
    qd, kd, vd = (torch.from_numpy(x.view(np.int16)).view(tdt).to(dev) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    dt_code = fa.FA_F16 if w.dtype == "f16" else fa.FA_BF16
    call_args = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                 w.B, w.H, w.Sq, w.Sk, w.D, float(w.scale), int(w.causal), dt_code)
    n_split = 0
    if w.split:
        n_split = fa.split_count(w.B, w.H, w.Sq, w.Sk, 0)
        ws_bytes = fa.split_workspace_size(w.B, w.H, w.Sq, w.Sk, w.D, 0)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        log(f"[bench] key split: {n_split} ranges, workspace {ws_bytes} bytes")

    def step():
        if w.split:
            st = fa.fa_fwd_split(*call_args, 0, ws.data_ptr(), ws_bytes, sp)
        else:
            st = fa.fa_fwd(*call_args, sp)
        if st != fa.FA_OK:
            raise fa.FaError(st)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # HIP events on the launch stream: one pair around the whole timed region
    # (throughput) and one pair around every launch (mean kernel duration for
    # the roofline; back-to-back launches, so the two agree to within the
    # event overhead)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    ms = ms_total / args.steps
    launch_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    ms_kernel = float(np.mean(launch_ms))
    flop = w.flops()
    tflops = flop / (ms * 1e-3) / 1e12
    tflops_kernel = flop / (ms_kernel * 1e-3) / 1e12
    gbs_kernel = w.io_bytes() / (ms_kernel * 1e-3) / 1e9
    log(f"[bench] {args.steps} steps: {ms:.4f} ms/step, {tflops:.1f} TFLOP/s; per launch "
        f"mean {ms_kernel:.4f} ms (min {min(launch_ms):.4f}, max {max(launch_ms):.4f}), "
        f"{tflops_kernel:.1f} TFLOP/s, {gbs_kernel:.0f} GB/s of algorithmic bytes (wall {wall:.3f} s)")

    # sampled parity of the timed output
    import oracle

    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, w.B * w.H * w.Sq - 1], rng.integers(0, w.B * w.H * w.Sq, 62)]))
    idx = torch.from_numpy(rows).to(dev)
    o_s = o.view(-1, w.D)[idx].double().cpu().numpy()
    l_s = lse.view(-1)[idx].double().cpu().numpy()
    threads = min(16, os.cpu_count() or 1)
    o_ref, l_ref = oracle.attention_rows(q, k, v, w.dtype, w.scale, w.causal, rows, threads=threads)
    err_o = float(np.abs(o_s - o_ref).max())
    err_l = float((np.abs(l_s - l_ref) / np.maximum(np.abs(l_ref), 1.0)).max())
    tol_o = 5e-3 if w.dtype == "f16" else 2e-2
    parity_ok = bool(err_o <= tol_o and err_l <= 1e-3 and np.isfinite(o_s).all())
    log(f"[bench] sampled parity: max|dO|={err_o:.2e} lse_rel={err_l:.2e} ok={parity_ok}")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {threads} threads, ~{args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(w, q, k, v, args.cpu_seconds, threads)

    traffic = traffic_for(w.name)
    line = {
        "metric": "attention fwd TFLOP/s and % of MI355X dense fp16/bf16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded i.i.d. normal Q, K, V)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Sq": w.Sq, "Sk": w.Sk, "D": w.D,
                   "causal": w.causal, "scale": w.scale, "algorithmic_flop": flop,
                   "algorithmic_bytes": w.io_bytes(), "key_split_ranges": n_split if w.split else None,
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * tflops / PEAK_TFLOPS_F16, 2),
        "roofline": ({"bound": "hbm", "achieved": round(gbs_kernel, 1), "peak": PEAK_HBM_GBS,
                      "unit": "GB/s", "frac": round(gbs_kernel / PEAK_HBM_GBS, 4),
                      "traffic": traffic, "kernel_ms": round(ms_kernel, 5),
                      "algorithmic_bytes_per_launch": w.io_bytes(),
                      "timed": "both kernels of a call (key ranges, then merge)"}
                     if w.split else
                     {"bound": "mfma", "achieved": round(tflops_kernel, 2), "peak": PEAK_TFLOPS_F16,
                      "unit": "TFLOP/s", "frac": round(tflops_kernel / PEAK_TFLOPS_F16, 4),
                      "traffic": traffic, "kernel_ms": round(ms_kernel, 5),
                      "algorithmic_flop_per_launch": flop}),
        "cpu_baseline": cpu,
        "parity_sample": {"rows": int(rows.size), "max_abs_err_o": err_o, "max_rel_err_lse": err_l,
                          "ok": parity_ok},
        "kernel_sha256_16": kernel_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
