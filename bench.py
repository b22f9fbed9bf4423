"""Benchmark of the fused attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--oracle auto|full|sample] [--all [attention|everything]]

One step is one fa_fwd call (the whole fused forward pass: scores, online
softmax, P.V, normalisation, lse) over the workload's seeded inputs, which are
resident in device memory before timing starts.  Prints one JSON line (with
--all, one line per workload, each with its own pass/fail status; a failing
workload does not stop the others).  The decode-shaped workloads (few queries,
long keys) run one fa_fwd_split call per step instead: the partial-result
kernel over the key ranges and the merge, with the workspace allocated before
timing.  The gemm_* workloads time one gemm_bias_gelu call per step (C =
gelu(A W^T + bias)), the softmax_* and rmsnorm_silu_* ones one row-kernel
call.

Reported alongside the throughput:
  * roofline: the dominant kernel against its roofline (dense fp16/bf16 MFMA
    peak, or HBM bandwidth for the decode, row-wise and merge kernels), with
    achieved = algorithmic work per launch / mean launch time measured with
    HIP events on the launch stream over the timed region; traffic = HBM
    bytes per launch from rocprofv3 counters when they were taken on the
    current kernel source (else null);
  * the GPU clock sampled during the timed region (AMD SMI GPU metrics), and
    the fraction of the peak at that clock;
  * cpu_baseline: the float64 oracle timed on the host's cores over the rows
    that the parity check compares (every row when that fits the time
    budget, else a seeded sample of distinct rows), plus one thread on the
    smallest workload as a per-core figure;
  * parity: the timed output against the oracle on those rows.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fa_inputs as fi  # noqa: E402

# MI355X dense MFMA peak for fp16/bf16: 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU.
PEAK_TFLOPS_F16 = 2516.6
PEAK_CLOCK_MHZ = 2400.0
# MI355X HBM3E peak bandwidth (8 TB/s).
PEAK_HBM_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "tile_level_programming_amd", "csrc", "fa_fwd.hip")
GEMM_SRC = os.path.join(ROOT, "tile_level_programming_amd", "csrc", "gemm_bias_gelu.hip")
ROWWISE_SRC = os.path.join(ROOT, "tile_level_programming_amd", "csrc", "rowwise.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
TOL_O = {"f16": 5e-3, "bf16": 2e-2}
TOL_LSE = 1e-3
SMALLEST = "tiny_b1h2_s128_d64_f16"


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


def counters_for(workload: str, src: str | None = None):
    """Matrix-unit busy share and LDS bank conflicts per launch, from the
    rocprofv3 counter passes of the workload's profile on this kernel source
    (counters are not collected in the timed run), or None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("kernel_sha256_16") != kernel_hash(src) or "mfma_busy_pct" not in ent:
        return None
    return {"mfma_busy_pct": ent["mfma_busy_pct"], "lds_bank_conflict_cycles": ent["lds_bank_conflict_cycles"],
            "lds_active_cycles": ent["lds_active_cycles"], "lds_conflict_rate": ent["lds_conflict_rate"],
            "source": ent.get("source")}


# --- the host: oracle threads, CPU model -------------------------------------


def oracle_threads() -> int:
    """Threads for the oracle: the process's CPU share.  OMP_NUM_THREADS when
    it is set (a machine that shares its host between GPUs sets it to one
    GPU's share), else every CPU this process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_fields(threads: int) -> dict:
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"cores": threads, "cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "cpus_allowed": affinity}


# --- the GPU clock during the timed region ------------------------------------


class ClockSampler:
    """Samples the graphics clock with AMD SMI (GPU metrics) on a side thread
    while the timed region runs.  The metrics table refreshes a few times a
    second, so a reading counts only once it shows the GPU busy (graphics
    activity >= 50%): the first readings of a region still describe the idle
    GPU before it.  The clock is the mean over the 8 XCDs' graphics clocks.
    Reports None when the metrics are not readable or never showed the load
    (the figure is then absent, never guessed)."""

    def __init__(self, period_s: float = 0.002):
        self.period = period_s
        self.samples = []
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        self._handle = None
        self._smi = None

    def _open(self):
        import amdsmi
        import torch

        amdsmi.amdsmi_init()
        self._smi = amdsmi
        handles = amdsmi.amdsmi_get_processor_handles()
        want = None
        try:
            p = torch.cuda.get_device_properties(0)
            want = (int(p.pci_domain_id), int(p.pci_bus_id), int(p.pci_device_id))
        except Exception:  # noqa: BLE001 - older torch: fall back to the only device
            pass
        for h in handles:
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
            dom, bus, rest = bdf.split(":")
            dev = rest.split(".")[0]
            if want is None or (int(dom, 16), int(bus, 16), int(dev, 16)) == want:
                self._handle = h
                break
        if self._handle is None and len(handles) == 1:
            self._handle = handles[0]
        if self._handle is None:
            raise RuntimeError("no AMD SMI device matches cuda:0")

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._handle)
        act = m.get("average_gfx_activity")
        if not isinstance(act, (int, float)) or act < 50:
            return None
        clks = m.get("current_gfxclks")
        if isinstance(clks, (list, tuple)):
            vals = [float(c) for c in clks if isinstance(c, (int, float)) and 0 < c < 10000]
            if vals:
                return sum(vals) / len(vals)
        c = m.get("current_gfxclk")
        if isinstance(c, (int, float)) and 0 < c < 10000:
            return float(c)
        c = m.get("average_gfxclk_frequency")
        if isinstance(c, (int, float)) and 0 < c < 10000:
            return float(c)
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
            except Exception as e:  # noqa: BLE001
                self.error = repr(e)
                return
            if v is not None:
                self.samples.append(v)
            time.sleep(self.period)

    def __enter__(self):
        try:
            self._open()
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        except Exception as e:  # noqa: BLE001
            self.error = repr(e)
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join(timeout=5)
        if self._smi is not None:
            try:
                self._smi.amdsmi_shut_down()
            except Exception:  # noqa: BLE001
                pass
        return False

    def result(self):
        if not self.samples:
            return {"mean_mhz": None, "samples": 0, "source": "AMD SMI GPU metrics",
                    "error": self.error or "no readable samples"}
        s = np.array(self.samples)
        return {"mean_mhz": round(float(s.mean()), 1), "median_mhz": round(float(np.median(s)), 1),
                "min_mhz": round(float(s.min()), 1), "max_mhz": round(float(s.max()), 1),
                "samples": int(s.size), "source": "AMD SMI GPU metrics: mean graphics clock of the 8 XCDs, "
                f"sampled every {self.period * 1e3:.0f} ms during the timed region, readings with graphics "
                "activity >= 50%"}


def peak_at_clock(peak: float, clock: dict):
    mhz = clock.get("median_mhz")
    return None if not mhz else peak * mhz / PEAK_CLOCK_MHZ


# --- timing -------------------------------------------------------------------


def time_steps(step, stream, steps, warmup: int):
    """W untimed warmup steps, then K timed steps on ``stream``: one event pair
    around the whole region and one around every launch.  K = None picks a
    count that makes the region about 2 s long (at least 200 steps, at most
    20000): the clock readings need a region of a second or more."""
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if steps is None:
        t0 = time.perf_counter()
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        per = (time.perf_counter() - t0) / 10
        steps = int(min(20000, max(200, 2.0 / max(per, 1e-7))))
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        start.record(stream)
        for e0, e1 in ev:
            e0.record(stream)
            step()
            e1.record(stream)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    launch_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    return ms, launch_ms, wall, clk.result(), steps


# Launches shorter than this are timed a second time from a captured HIP graph:
# back-to-back launches from the host leave the GPU idle between such short
# kernels, so the host's call rate, not the kernel, would set the step time.
GRAPH_BELOW_MS = 0.1
GRAPH_LAUNCHES = 100  # launches per captured graph


def time_steps_graph(launch, steps: int):
    """``steps`` calls of ``launch(stream_handle)`` replayed from HIP graphs of
    GRAPH_LAUNCHES calls each (plus one graph for the remainder), timed with one
    event pair around all the replays.  The graphs hold kernel launches only
    (no memory-set nodes).  Returns ms per step."""
    import torch

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sp = torch.cuda.current_stream().cuda_stream
            for _ in range(n):
                launch(sp)
        return g

    full, rest = divmod(steps, GRAPH_LAUNCHES)
    g_full = capture(GRAPH_LAUNCHES) if full else None
    g_rest = capture(rest) if rest else None
    for g in (g_full, g_rest):
        if g is not None:
            g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(full):
        g_full.replay()
    if g_rest is not None:
        g_rest.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


# --- the oracle on the host ------------------------------------------------------


def visible_keys(w, rows: np.ndarray) -> np.ndarray:
    """Keys each flat query row sees (top-left causal mask, or all)."""
    if not w.causal:
        return np.full(rows.size, w.Sk, dtype=np.int64)
    return np.minimum(rows % w.Sq, w.Sk - 1) + 1


def oracle_rows_plan(w, q, k, v, mode: str, seconds: float, threads: int, rng):
    """The rows the oracle evaluates: all of them (mode 'full', or 'auto' when
    the calibrated estimate fits twice the budget), else distinct seeded rows
    sized to the budget.  Returns (rows, description)."""
    import oracle

    total = w.B * w.H * w.Sq
    if mode == "full":
        return np.arange(total, dtype=np.int64), "every row"
    # calibrate: distinct random rows, growing until a batch takes >= 1 s
    n = min(total, threads * 4)
    while True:
        rows = np.sort(rng.choice(total, size=n, replace=False))
        t0 = time.perf_counter()
        oracle.attention_rows(q, k, v, w.dtype, w.scale, w.causal, rows, threads=threads)
        dt = time.perf_counter() - t0
        if dt >= 1.0 or n >= total:
            break
        n = min(total, n * 4)
    per_pair = dt / max(1, int(visible_keys(w, rows).sum()))
    full_est = per_pair * w.unmasked_pairs() * w.B * w.H
    if mode == "auto" and full_est <= 2 * seconds:
        return np.arange(total, dtype=np.int64), f"every row (estimated {full_est:.0f} s)"
    n = int(min(total, max(threads, seconds / max(per_pair * w.Sk, 1e-12))))
    rows = np.sort(rng.choice(total, size=n, replace=False))
    return rows, f"{n} distinct seeded random rows ({n / total:.2%} of the rows)"


def per_core_figure(threads_note: str):
    """One oracle thread on the smallest workload, repeated for >= 1 s."""
    import oracle

    w = fi.WORKLOADS[SMALLEST]
    q, k, v = fi.make_inputs(w)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.attention(q, k, v, w.dtype, w.scale, w.causal, threads=1)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 1.0:
            break
    return {"value": round(reps * w.flops() / dt / 1e12, 6), "unit": "TFLOP/s", "threads": 1,
            "sample": f"{reps} full passes over {w.name} (all {w.B * w.H * w.Sq} rows), float64, one thread, "
                      f"{dt:.2f} s wall{threads_note}"}


def lse_stats(l_gpu, l_ref):
    d = np.abs(l_gpu - l_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        unguarded = d / np.abs(l_ref)
    return {
        "max_rel_err_lse": float((d / np.maximum(np.abs(l_ref), 1.0)).max()),
        "max_rel_err_lse_unguarded": float(np.nanmax(unguarded)) if unguarded.size else 0.0,
        "max_abs_err_lse": float(d.max()),
        "rows_lse_ref_below_1": int((np.abs(l_ref) < 1).sum()),
    }


# --- attention workloads ------------------------------------------------------------


def run_attention(args, w):
    import torch

    from tile_level_programming_amd import fa

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

    def launch(stream_handle):
        if w.split:
            st = fa.fa_fwd_split(*call_args, 0, ws.data_ptr(), ws_bytes, stream_handle)
        else:
            st = fa.fa_fwd(*call_args, stream_handle)
        if st != fa.FA_OK:
            raise fa.FaError(st)

    def step():
        launch(sp)

    log(f"[bench] warmup {args.warmup}, then {args.steps or 'about 2 s of'} timed steps")
    ms, launch_ms, wall, clock, steps = time_steps(step, stream, args.steps, args.warmup)
    ms_kernel = float(np.mean(launch_ms))
    graph = None
    if not w.split and ms_kernel < GRAPH_BELOW_MS:
        # the same steps again from captured graphs; the output of the
        # replays must equal that of an eager call bit for bit
        ref_o, ref_l = o.clone(), lse.clone()
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        ms_graph = time_steps_graph(launch, steps)
        same = bool(torch.equal(o.view(torch.int16), ref_o.view(torch.int16))
                    and torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)))
        log(f"[bench] {steps} steps from HIP graphs of {GRAPH_LAUNCHES} launches: {ms_graph:.4f} ms/step "
            f"(launched from the host: {ms:.4f}); output equal to the eager call's: {same}")
        if not same:
            raise RuntimeError("graph replays changed the output")
        graph = {"ms_per_step": round(ms_graph, 5), "launches_per_graph": GRAPH_LAUNCHES,
                 "host_launched_ms_per_step": round(ms, 5)}
        ms = ms_graph
    flop = w.flops()
    tflops = flop / (ms * 1e-3) / 1e12
    tflops_kernel = flop / (ms_kernel * 1e-3) / 1e12
    gbs_kernel = w.io_bytes() / (ms_kernel * 1e-3) / 1e9
    log(f"[bench] {steps} steps: {ms:.4f} ms/step, {tflops:.1f} TFLOP/s; per launch "
        f"mean {ms_kernel:.4f} ms (min {min(launch_ms):.4f}, max {max(launch_ms):.4f}), "
        f"{tflops_kernel:.1f} TFLOP/s, {gbs_kernel:.0f} GB/s of algorithmic bytes (wall {wall:.3f} s); "
        f"clock {clock.get('median_mhz')} MHz")

    line = {
        "metric": "attention fwd TFLOP/s and % of MI355X dense fp16/bf16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded i.i.d. normal Q, K, V)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Sq": w.Sq, "Sk": w.Sk, "D": w.D,
                   "causal": w.causal, "scale": w.scale, "sigma_qk": w.sigma_qk, "algorithmic_flop": flop,
                   "algorithmic_bytes": w.io_bytes(), "key_split_ranges": n_split if w.split else None,
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * tflops / PEAK_TFLOPS_F16, 2),
        "clock": clock,
    }
    if graph is not None:
        line["timing"] = {"steps_from": "HIP graphs (launches shorter than the host's call rate)", **graph}
    traffic = traffic_for(w.name)
    if w.split:
        line["roofline"] = {"bound": "hbm", "achieved": round(gbs_kernel, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(gbs_kernel / PEAK_HBM_GBS, 4), "traffic": traffic,
                            "kernel_ms": round(ms_kernel, 5), "algorithmic_bytes_per_launch": w.io_bytes(),
                            "timed": "both kernels of a call (key ranges, then merge)"}
    else:
        pk = peak_at_clock(PEAK_TFLOPS_F16, clock)
        line["pct_of_peak_at_measured_clock"] = round(100.0 * tflops / pk, 2) if pk else None
        line["roofline"] = {"bound": "mfma", "achieved": round(tflops_kernel, 2), "peak": PEAK_TFLOPS_F16,
                            "unit": "TFLOP/s", "frac": round(tflops_kernel / PEAK_TFLOPS_F16, 4),
                            "frac_at_measured_clock": round(tflops_kernel / pk, 4) if pk else None,
                            "traffic": traffic, "kernel_ms": round(ms_kernel, 5),
                            "algorithmic_flop_per_launch": flop}
    line["counters"] = counters_for(w.name)
    line["kernel_sha256_16"] = kernel_hash()
    if args.no_check:
        line["cpu_baseline"] = None
        line["parity"] = None
        return line

    # the oracle on the host: the same rows are the cpu baseline and the
    # parity check of the timed output
    import oracle

    threads = oracle_threads()
    rng = np.random.default_rng(1234)
    rows, how = oracle_rows_plan(w, q, k, v, args.oracle, args.cpu_seconds, threads, rng)
    log(f"[bench] oracle on {threads} threads over {how}")
    t0 = time.perf_counter()
    o_ref, l_ref = oracle.attention_rows(q, k, v, w.dtype, w.scale, w.causal, rows, threads=threads)
    dtc = time.perf_counter() - t0
    idx = torch.from_numpy(rows).to(dev)
    o_s = o.view(-1, w.D)[idx].double().cpu().numpy()
    l_s = lse.view(-1)[idx].double().cpu().numpy()
    err = np.abs(o_s - o_ref)
    err_o = float(err.max())
    where = int(rows[np.unravel_index(np.argmax(err), err.shape)[0]])
    ls = lse_stats(l_s, l_ref)
    tol_o = TOL_O[w.dtype]
    parity_ok = bool(err_o <= tol_o and ls["max_rel_err_lse"] <= TOL_LSE and np.isfinite(o_s).all()
                     and np.isfinite(l_s).all())
    log(f"[bench] parity over {rows.size} rows: max|dO|={err_o:.2e} lse={ls['max_rel_err_lse']:.2e} ok={parity_ok}")
    row_flop = int(4 * w.D * visible_keys(w, rows).sum())
    cpu = {
        "value": round(row_flop / dtc / 1e12, 6),
        "unit": "TFLOP/s",
        **host_fields(threads),
        "kind": "oracle",
        "sample": f"{how} of {w.name}: {rows.size} of {w.B * w.H * w.Sq} query rows, float64, explicit scores "
                  f"over all {w.Sk} keys per row, {dtc:.1f} s wall on {threads} threads; value = the rows' "
                  f"algorithmic FLOP / wall time",
    }
    if not args.no_per_core:
        cpu["per_core"] = per_core_figure("")
    line["cpu_baseline"] = cpu
    line["parity"] = {"rows": int(rows.size), "of_rows": w.B * w.H * w.Sq, "max_abs_err_o": err_o,
                      "bar_o": tol_o, "worst_row": where, **ls, "bar_lse": TOL_LSE, "ok": parity_ok}
    return line


# --- GEMM + bias + GELU ---------------------------------------------------------------


def run_gemm(args, w):
    """One step = one gemm_bias_gelu call: C = gelu(A W^T + bias)."""
    import torch

    import oracle.gemm as og
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

    ms, launch_ms, wall, clock, steps = time_steps(step, stream, args.steps, args.warmup)
    ms_kernel = float(np.mean(launch_ms))
    flop = w.flops()
    tflops = flop / (ms * 1e-3) / 1e12
    tflops_kernel = flop / (ms_kernel * 1e-3) / 1e12
    log(f"[bench] {steps} steps: {ms:.4f} ms/step, {tflops:.1f} TFLOP/s; per launch mean {ms_kernel:.4f} ms "
        f"(min {min(launch_ms):.4f}, max {max(launch_ms):.4f}), {tflops_kernel:.1f} TFLOP/s")

    if args.no_check:
        return {"metric": "GEMM + bias + GELU TFLOP/s", "value": round(tflops, 2), "unit": "TFLOP/s",
                "ms_per_step": round(ms, 5), "config": {"workload": w.name}, "clock": clock,
                "roofline": {"achieved": round(tflops_kernel, 2), "kernel_ms": round(ms_kernel, 5)},
                "parity": None, "cpu_baseline": None, "kernel_sha256_16": kernel_hash(GEMM_SRC)}
    # rows the oracle evaluates (all columns of each): two seeded rows in
    # every 256-row block (so every output tile is checked), then more
    # distinct random rows up to the time budget; they are both the cpu
    # baseline and the parity check
    threads = oracle_threads()
    rng = np.random.default_rng(7)
    blocks = np.arange(0, w.M, 256)
    base = np.unique(np.concatenate([[0, w.M - 1], blocks + rng.integers(0, 256, blocks.size),
                                     blocks + rng.integers(0, 256, blocks.size)]))
    base = base[base < w.M]
    t0 = time.perf_counter()
    ref0 = og.gemm_rows(a, wt, b, w.dtype, rows=base, threads=threads)
    dt0 = time.perf_counter() - t0
    per_row = dt0 / base.size
    rest = np.setdiff1d(np.arange(w.M), base)
    n_more = int(min(rest.size, max(0, (args.cpu_seconds - dt0) / max(per_row, 1e-9))))
    more = np.sort(rng.choice(rest, size=n_more, replace=False)) if n_more else np.zeros(0, np.int64)
    t0 = time.perf_counter()
    ref1 = og.gemm_rows(a, wt, b, w.dtype, rows=more, threads=threads) if n_more else np.zeros((0, w.N))
    dt1 = time.perf_counter() - t0
    rows = np.concatenate([base, more])
    ref = np.concatenate([ref0, ref1])
    cs = c[torch.from_numpy(rows).to(dev)].double().cpu().numpy()
    rel = 2.0 ** -10 if w.dtype == "f16" else 2.0 ** -7
    err = float((np.abs(cs - ref) / np.maximum(np.abs(ref), 1.0)).max())
    parity_ok = bool(err <= rel and np.isfinite(cs).all())
    log(f"[bench] parity over {rows.size} rows: max |dC|/max(|C|,1) = {err:.2e} (bar {rel:.2e}) ok={parity_ok}")
    dtc = dt0 + dt1
    cpu = {"value": round(rows.size * 2 * w.N * w.K / dtc / 1e12, 6), "unit": "TFLOP/s", **host_fields(threads),
           "kind": "oracle",
           "sample": f"{rows.size} distinct output rows of {w.name} ({rows.size / w.M:.2%} of the rows, all {w.N} "
                     f"columns each; two in every 256-row block, the rest seeded random), float64, {dtc:.1f} s wall "
                     f"on {threads} threads"}
    pk = peak_at_clock(PEAK_TFLOPS_F16, clock)
    return {
        "metric": "GEMM + bias + GELU TFLOP/s and % of MI355X dense fp16/bf16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
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
        "pct_of_peak_at_measured_clock": round(100.0 * tflops / pk, 2) if pk else None,
        "clock": clock,
        "roofline": {"bound": "mfma", "achieved": round(tflops_kernel, 2), "peak": PEAK_TFLOPS_F16,
                     "unit": "TFLOP/s", "frac": round(tflops_kernel / PEAK_TFLOPS_F16, 4),
                     "frac_at_measured_clock": round(tflops_kernel / pk, 4) if pk else None,
                     "traffic": traffic_for(w.name, GEMM_SRC), "kernel_ms": round(ms_kernel, 5),
                     "algorithmic_flop_per_launch": flop},
        "cpu_baseline": cpu,
        "parity": {"rows": int(rows.size), "of_rows": w.M, "max_rel_err": err, "bar": rel, "ok": parity_ok},
        "kernel_sha256_16": kernel_hash(GEMM_SRC),
    }


# --- row-wise kernels --------------------------------------------------------------------


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

    def launch(stream_handle):
        if w.op == "softmax":
            st = fa.row_softmax(xd.data_ptr(), y.data_ptr(), w.R, w.C, dt_code, stream_handle)
        else:
            st = fa.rmsnorm_silu(xd.data_ptr(), gd.data_ptr(), y.data_ptr(), w.R, w.C, w.eps, dt_code, stream_handle)
        if st != fa.FA_OK:
            raise fa.FaError(st)

    def step():
        launch(sp)

    ms, launch_ms, wall, clock, steps = time_steps(step, stream, args.steps, args.warmup)
    ms_kernel = float(np.mean(launch_ms))
    timing = None
    if ms_kernel < GRAPH_BELOW_MS:
        ref_y = y.clone()
        y.fill_(float("nan"))
        ms_graph = time_steps_graph(launch, steps)
        same = bool(torch.equal(y.view(torch.int16), ref_y.view(torch.int16)))
        log(f"[bench] {steps} steps from HIP graphs of {GRAPH_LAUNCHES} launches: {ms_graph:.4f} ms/step "
            f"(launched from the host: {ms:.4f}); output equal to the eager call's: {same}")
        if not same:
            raise RuntimeError("graph replays changed the output")
        timing = {"steps_from": "HIP graphs (launches shorter than the host's call rate)",
                  "ms_per_step": round(ms_graph, 5), "launches_per_graph": GRAPH_LAUNCHES,
                  "host_launched_ms_per_step": round(ms, 5)}
        ms = ms_graph
    nbytes = w.io_bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    gbs_kernel = nbytes / (ms_kernel * 1e-3) / 1e9
    log(f"[bench] {steps} steps: {ms:.4f} ms/step, {gbs:.0f} GB/s; per launch mean {ms_kernel:.4f} ms "
        f"(min {min(launch_ms):.4f}, max {max(launch_ms):.4f}), {gbs_kernel:.0f} GB/s")

    if args.no_check:
        return {"metric": f"{w.op} GB/s", "value": round(gbs, 1), "unit": "GB/s", "ms_per_step": round(ms, 5),
                "config": {"workload": w.name}, "clock": clock, "timing": timing,
                "roofline": {"achieved": round(gbs_kernel, 1), "kernel_ms": round(ms_kernel, 5)},
                "parity": None, "cpu_baseline": None, "kernel_sha256_16": kernel_hash(ROWWISE_SRC)}
    # every row through the oracle: both the parity check and the cpu baseline
    threads = oracle_threads()
    t0 = time.perf_counter()
    ref = (orw.softmax_rows(x, w.dtype, threads=threads) if w.op == "softmax"
           else orw.rmsnorm_silu_rows(x, g, w.dtype, w.eps, threads=threads))
    dtc = time.perf_counter() - t0
    ys = y.double().cpu().numpy()
    rel = 2.0 ** -10 if w.dtype == "f16" else 2.0 ** -7
    floor = (2.0 ** -24 if w.dtype == "f16" else 1e-30) if w.op == "softmax" else 1e-5
    over = float((np.abs(ys - ref) - (rel * np.abs(ref) + floor)).max())
    parity_ok = bool(over <= 0 and np.isfinite(ys).all())
    log(f"[bench] parity over all {w.R} rows: max (|dy| - bar) = {over:.2e} ok={parity_ok}")
    cpu = {"value": round(nbytes / dtc / 1e9, 3), "unit": "GB/s", **host_fields(threads), "kind": "oracle",
           "sample": f"every row of {w.name} ({w.R} rows), float64, {dtc:.2f} s wall on {threads} threads; value = "
                     "the workload's algorithmic bytes / wall time"}
    return {
        "metric": f"{w.op} GB/s of algorithmic bytes and % of MI355X HBM peak",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded i.i.d. normal rows" + (", normal weight)" if g is not None else ")"),
        "config": {"workload": w.name, "op": w.op, "R": w.R, "C": w.C, "algorithmic_bytes": nbytes,
                   "parallelism": "single GPU"},
        "clock": clock,
        "timing": timing,
        "roofline": {"bound": "hbm", "achieved": round(gbs_kernel, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs_kernel / PEAK_HBM_GBS, 4), "traffic": traffic_for(w.name, ROWWISE_SRC),
                     "kernel_ms": round(ms_kernel, 5), "algorithmic_bytes_per_launch": nbytes},
        "cpu_baseline": cpu,
        "parity": {"rows": w.R, "of_rows": w.R, "max_excess_over_bar": over, "ok": parity_ok},
        "kernel_sha256_16": kernel_hash(ROWWISE_SRC),
    }


def run_one(args, name):
    if name in fi.GEMM_WORKLOADS:
        return run_gemm(args, fi.GEMM_WORKLOADS[name])
    if name in fi.ROW_WORKLOADS:
        return run_rows(args, fi.ROW_WORKLOADS[name])
    return run_attention(args, fi.ALL_WORKLOADS[name])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: enough for about 2 s, at least 200)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=fi.HEADLINE, choices=list(fi.ALL_WORKLOADS) + list(fi.GEMM_WORKLOADS)
                    + list(fi.ROW_WORKLOADS))
    ap.add_argument("--all", nargs="?", const="attention", choices=["attention", "everything"], default=None,
                    help="run every attention workload (or every workload of every entry point) and print one "
                         "line per workload with its pass/fail status; a failure does not stop the others")
    ap.add_argument("--oracle", choices=["auto", "full", "sample"], default="auto",
                    help="rows the oracle checks: every row (full), a seeded sample sized to --cpu-seconds "
                         "(sample), or every row when that is estimated to fit twice that budget (auto)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-per-core", action="store_true", help="skip the one-thread oracle figure")
    ap.add_argument("--no-check", action="store_true",
                    help="time only: no oracle (parity and cpu_baseline null), for profiler runs")
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

    from tile_level_programming_amd import fa  # noqa: F401 - fails loudly when the library is missing

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: 10 copies of {n} bytes (read {n} B + write {n} B each)")
        return

    if args.all is None:
        print(json.dumps(run_one(args, args.workload)), flush=True)
        return

    names = list(fi.WORKLOADS)
    if args.all == "everything":
        names += list(fi.DECODE_WORKLOADS) + list(fi.GEMM_WORKLOADS) + list(fi.ROW_WORKLOADS)
    failed = 0
    for name in names:
        try:
            line = run_one(args, name)
            line["status"] = ("timed, not checked" if line["parity"] is None else
                              "pass" if line["parity"]["ok"] else "fail: parity")
        except Exception as e:  # noqa: BLE001 - record and go on to the next workload
            line = {"config": {"workload": name}, "status": f"error: {type(e).__name__}: {e}"}
            torch.cuda.synchronize()
        failed += not (line["status"] == "pass" or line["status"] == "timed, not checked")
        print(json.dumps(line), flush=True)
        del line
        torch.cuda.empty_cache()
    log(f"[bench] --all: {len(names) - failed} of {len(names)} workloads passed")
    sys.exit(1 if failed else 0)


if __name__ == "__main__":
    main()
