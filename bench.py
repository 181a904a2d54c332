#!/usr/bin/env python3
"""Benchmark of the FP8 attention hot path on one MI355X.

One step = one pass of the whole path over the workload's synthetic inputs,
which are resident in HBM before timing starts: fp8attn_quantize (stats,
finalize, pack) followed by fp8attn_forward.  The plan (segment schedule) is
built once beforehand, as it is reused across calls.

Timing: W untimed warmup steps, then K timed steps bracketed by
torch.cuda.synchronize(); ``value`` is the step throughput over those K steps,
and HIP events recorded on the launch stream around every forward give the
attention kernel's average launch duration for the roofline.  Then the
protocol of sglang PR "[diffusion] attention: add fp8_fa_sm120 FP8 backend for
SM120 GPUs" ("Speed Tests and Profiling": kernel only, CUDA events, 20 warmup,
5 x 10 iterations) is run on its own for the forward, the quantize and the
whole step: 20 warmup launches, then 5 repetitions of 10 back-to-back
launches, reporting the median of the five per-launch means with the min and
max.  The shader clock is sampled (amdsmi GPU metrics) while the protocol's
forward launches run.

Prints one JSON line.  FLOPs are counted as 4 * sum(L^2) * H * D.

``--fmt mxfp4`` times the block-scaled FP4 variant instead and reports it
against the FP4 matrix-core peak; ``--q-centre`` adds Q block-mean centring
(either format); the default line is the E4M3 path.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 attn TFLOP/s (4*S^2*H*D) at S=30272 H=56 D=128; % of FP8 MFMA peak"
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense FP8 MFMA (published)
FP4_PEAK_TFLOPS = 10100.0       # MI355X dense FP4 MFMA (published)
METRIC_FP4 = "FP4 attn TFLOP/s (4*S^2*H*D), block-scaled E2M1 operands; % of FP4 MFMA peak"
METRIC_CAUSAL = "FP8 causal attn TFLOP/s (2*S*(S+1)*H*D, visible pairs only); % of FP8 MFMA peak"
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "s30272_h56_koffset"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attention_counters.json")


def l2_stream_bytes(items, segments, bm, wg_per_cu, key_bytes, q_row_bytes, out_bytes,
                    causal=False, cus_per_xcd=32, xcds=8, kbn=64):
    """Bytes a forward launch must move between HBM and the eight per-XCD L2
    caches when the concurrent workgroups of an XCD walk the K/V tiles of a
    (segment, head) together: each round of an XCD's workgroups reads the K/V
    tiles of every (segment, head) it touches once, and every item (or key
    piece) reads its own Q tile once; the output is written once.

    items: the plan's launch-ordered work list, (segment, q0, head, split) with
    split = piece | count << 4 | slot << 8 (0: whole item); launch position p
    runs on XCD p % xcds as the (p // xcds)-th workgroup there.
    key_bytes: K plus V bytes per key and head; q_row_bytes: Q bytes per query
    row and head; out_bytes: output bytes per launch.
    """
    slots = wg_per_cu * cus_per_xcd
    rounds = {}
    q_bytes = 0
    for p, (seg, q0, head, split) in enumerate(items):
        if seg < 0:
            continue
        L = segments[seg]
        nkt = (L + kbn - 1) // kbn
        hi = ((min(L, q0 + bm) + kbn - 1) // kbn) if causal else nkt
        lo = 0
        if split:
            i, n = split & 15, (split >> 4) & 15
            lo, hi = nkt * i // n, nkt * (i + 1) // n
        tiles = rounds.setdefault((p % xcds, (p // xcds) // slots), {}).setdefault((seg, head), set())
        tiles.update(range(lo, hi))
        q_bytes += bm * q_row_bytes
    kv = sum(len(t) for r in rounds.values() for t in r.values()) * kbn * key_bytes
    return int(kv + q_bytes + out_bytes)


def kernel_source_hash(kernel_file: str = "attention.hip") -> str:
    """sha256 (16 hex) of the attention kernel's code with comments and blank lines
    removed, so that counters stay attached to the code they were taken on."""
    h = hashlib.sha256()
    for f in (kernel_file, "internal.h"):
        with open(os.path.join(ROOT, "fp8_flash_attention_amd", "csrc", f)) as fh:
            t = fh.read()
        t = re.sub(r"/\*.*?\*/", "", t, flags=re.S)
        t = re.sub(r"//[^\n]*", "", t)
        h.update("\n".join(l.rstrip() for l in t.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def measured_traffic(key: str, kernel_file: str = "attention.hip"):
    """HBM bytes per attention launch from committed rocprofv3 counters, if they were
    taken on the current kernel source; else None."""
    try:
        with open(COUNTERS_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(key)
    if not e or e.get("kernel_hash") != kernel_source_hash(kernel_file):
        return None
    return e.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class ClockSampler:
    """Samples the GPU shader clock (MHz) from amdsmi GPU metrics on a host thread
    while GPU work runs; reports nothing if amdsmi is not usable."""

    def __init__(self, index: int = 0, period_s: float = 0.005):
        import threading
        self.period = period_s
        self.samples = []
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        self._h = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[index]
            self._read()
            self.samples.clear()
        except Exception as e:  # noqa: BLE001 - report, do not fail the bench
            self.error = f"{type(e).__name__}: {e}"
            self._h = None
        self._threading = threading

    def _read(self):
        """(metrics timestamp, MHz) of the current metrics table, or None."""
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._h)
        ts = m.get("system_clock_counter")
        vals = m.get("current_gfxclks")
        if isinstance(vals, (list, tuple)):
            vals = [v for v in vals if isinstance(v, (int, float)) and 0 < v < 10000]
            if vals:
                return ts, sum(vals) / len(vals)
        v = m.get("current_gfxclk")
        return (ts, float(v)) if isinstance(v, (int, float)) and 0 < v < 10000 else None

    def _run(self):
        seen = set()
        while not self._stop.is_set():
            try:
                r = self._read()
                # keep one sample per refresh of the metrics table: the driver
                # updates it far less often than this thread reads it
                if r is not None and (r[0] is None or r[0] not in seen):
                    seen.add(r[0])
                    self.samples.append(r[1])
            except Exception as e:  # noqa: BLE001
                self.error = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self.period)

    def __enter__(self):
        if self._h is not None:
            self._thread = self._threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        return False

    def summary(self):
        if len(self.samples) < 2:
            return {"samples": len(self.samples), "error": self.error or
                    "the metrics table was not refreshed during the timed region"}
        # samples taken while the GPU idled (before the first launch, between
        # repetitions) read the idle clock: keep those above half the highest
        top = max(self.samples)
        v = sorted(x for x in self.samples if x >= 0.5 * top)
        pct = lambda f: round(v[min(len(v) - 1, int(f * len(v)))], 0)   # noqa: E731
        return {"median_mhz": pct(0.5), "p05_mhz": pct(0.05), "p95_mhz": pct(0.95), "samples": len(v),
                "idle_samples_dropped": len(self.samples) - len(v),
                "source": "amdsmi gpu_metrics current_gfxclks (mean over XCDs), one sample per refresh "
                          "of the metrics table (polled every 5 ms)"}


def protocol(fn, stream, warmup: int = 20, reps: int = 5, per: int = 10):
    """20 warmup launches, then `reps` x `per` back-to-back launches timed with events
    on `stream`: median, min and max of the per-launch means (milliseconds)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    means = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(per):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        means.append(e0.elapsed_time(e1) / per)
    v = sorted(means)
    return {"median_ms": round(v[len(v) // 2], 4), "min_ms": round(v[0], 4), "max_ms": round(v[-1], 4),
            "reps_ms": [round(x, 4) for x in means], "warmup": warmup, "reps": reps, "per_rep": per}


def cpu_baseline(w, q, k, v, budget_s: float):
    """The float64 oracle on a bounded sample of query rows (all heads), in TFLOP/s."""
    import torch
    from oracle import attention as A
    from workloads import sample_rows

    threads = torch.get_num_threads()
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    seg = w.segments
    cu = w.cu_seqlens
    rows_done, flops, t0 = 0, 0.0, time.time()
    batch = 32
    pool = sample_rows(w.tokens, 4096, seed=w.seed + 11)
    while rows_done < len(pool):
        rows = pool[rows_done: rows_done + batch]
        A.attention_rows(qc, kc, vc, cu, w.softmax_scale, rows)
        for r in rows:
            s = max(i for i in range(len(seg)) if cu[i] <= r)
            flops += 4.0 * seg[s] * w.heads * w.head_dim
        rows_done += len(rows)
        if time.time() - t0 >= budget_s:
            break
    dt = time.time() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"float64 oracle on {rows_done} seeded query rows x {w.heads} heads of {w.name} "
                      f"({dt:.1f} s wall; quantization not included)"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-skeleton", action="store_true", help="skip the MFMA-only skeleton runs (profiling)")
    ap.add_argument("--fmt", choices=("e4m3", "mxfp4"), default="e4m3",
                    help="operand format: the E4M3 path (default) or the block-scaled FP4 variant")
    ap.add_argument("--q-centre", action="store_true",
                    help="centre Q by its 128-row block means (E4M3: mean term from a precomputed table)")
    ap.add_argument("--exact-probs", action="store_true",
                    help="e4m3: probabilities rounded from the FP32 exp2 instead of the log-linear code")
    ap.add_argument("--causal", action="store_true",
                    help="causal plan (FLOPs then count the visible pairs, 2 * sum L(L+1) * H * D)")
    ap.add_argument("--lse", action="store_true", help="the forward also writes the LSE output")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after timing, run one plain device copy of BYTES bytes (a known-size "
                         "reference dispatch for scaling HBM traffic counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); the path shards by "
              "heads across GPUs with no exchange inside attention, but no multi-GPU launch is implemented.",
              file=sys.stderr)
        return 2

    import torch
    import fp8_flash_attention_amd as fa
    from workloads import WORKLOADS, generate

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    q, k, v = generate(w, device="cuda")
    mx = args.fmt == "mxfp4"
    plan = fa.Plan(w.tokens, w.heads, w.cu_seqlens, w.softmax_scale, device=0, fmt=args.fmt,
                   q_centre=args.q_centre, causal=args.causal, head_dim=w.head_dim,
                   exact_probs=args.exact_probs and not mx)
    ws = plan.new_workspace()
    out = torch.empty((w.tokens, w.heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.heads, w.tokens), dtype=torch.float32, device=dev) if args.lse else None
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        fa.quantize(plan, q, k, v, ws)
        if ev is not None:
            ev[0].record(stream)
        fa.forward(plan, ws, out, lse)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    qev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        qev[i][0].record(stream)
        step(evs[i])
        qev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    fwd_ms = [a.elapsed_time(b) for a, b in evs]
    step_ms = [a.elapsed_time(b) for a, b in qev]

    # the pages' kernel-only protocol, separately for the forward (with the
    # shader clock sampled meanwhile), the quantize and the whole step
    fwd_proto = protocol(lambda: fa.forward(plan, ws, out, lse), stream)
    # the shader clock while the forward runs: the driver refreshes its metrics
    # table only every so often, so sample over a sustained run of forward
    # launches (about 3 s, after the timed protocol) rather than the short
    # timed windows
    sampler = ClockSampler(0)
    n_clock = min(20000, max(1, int(3000.0 / max(fwd_proto["median_ms"], 1e-3))))
    with sampler:
        for _ in range(n_clock):
            fa.forward(plan, ws, out, lse)
        torch.cuda.synchronize()
    sclk = dict(sampler.summary(), window_launches=n_clock)
    quant_proto = protocol(lambda: fa.quantize(plan, q, k, v, ws), stream)
    step_proto = protocol(step, stream)
    ms_step = wall * 1e3 / args.steps
    ms_fwd = sum(fwd_ms) / len(fwd_ms)
    ms_quant = sum(s - f for s, f in zip(step_ms, fwd_ms)) / len(fwd_ms)
    flops = (2.0 * sum(L * (L + 1) for L in w.segments) * w.heads * w.head_dim) if args.causal else w.flops
    value = flops / (ms_step * 1e-3) / 1e12
    fwd_tflops = flops / (ms_fwd * 1e-3) / 1e12

    # MFMA-only skeletons: measured matrix-core ceilings and shader clocks, with a
    # fixed operand pattern (short run) and with rotating random E4M3 operands long
    # enough (~30 ms) for the clock to settle where random data holds it
    from fp8_flash_attention_amd import _lib
    import ctypes

    def skeleton_run(iters, random_operands):
        tf, mhz = ctypes.c_double(), ctypes.c_double()
        rc = _lib.lib().fp8attn_mfma_peak(0, iters, random_operands, ctypes.byref(tf), ctypes.byref(mhz))
        return {"tflops": round(tf.value, 1), "sclk_mhz": round(mhz.value, 0)} if rc == 0 else None

    skeleton = None if args.no_skeleton or mx else skeleton_run(2000, 0)
    skeleton_random = None if args.no_skeleton or mx else skeleton_run(100000, 1)

    peak = FP4_PEAK_TFLOPS if mx else FP8_PEAK_TFLOPS
    kfile = "attention_mx.hip" if mx else "attention.hip"
    key = (w.name + (":mxfp4" if mx else "") + (":qc" if args.q_centre else "") + (":causal" if args.causal else "")
           + (":exact" if args.exact_probs and not mx else "") + (":lse" if args.lse else ""))
    traffic = measured_traffic(key, kfile)
    info = plan.info()
    kw = 64 if w.head_dim <= 64 and not mx else 128      # channels the kernel reads per row
    l2_floor = None if args.q_centre else l2_stream_bytes(
        plan.work_items(), list(w.segments), info["query_tile"], 1 if info["query_tile"] == 256 and not mx else 2,
        key_bytes=2 * (kw // 2 + kw // 32) if mx else 2 * kw, q_row_bytes=(kw // 2 + kw // 32) if mx else kw,
        out_bytes=2 * w.tokens * w.heads * w.head_dim, causal=args.causal,
        cus_per_xcd=torch.cuda.get_device_properties(dev).multi_processor_count // 8)
    res = {
        "metric": (METRIC_FP4 if mx else (METRIC_CAUSAL if args.causal else METRIC)) + (
            " [causal: visible pairs only]" if mx and args.causal else "") + (
            f" [head_dim {w.head_dim}]" if w.head_dim != 128 else ""),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4e2m1" if mx else "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "heads": w.heads, "head_dim": w.head_dim,
                   "cu_seqlens": list(w.cu_seqlens), "seed": w.seed, "softmax_scale": w.softmax_scale,
                   "k_offset_var": w.k_offset_var, "step": "quantize + forward",
                   **({"q_offset_var": w.q_offset_var} if w.q_offset_var is not None else {}),
                   **({"format": "mxfp4"} if mx else {}),
                   **({"q_centre": True} if args.q_centre else {}),
                   **({"causal": True} if args.causal else {}),
                   **({"lse": True} if args.lse else {}),
                   **({} if mx else {"probabilities": "exact exp2" if args.exact_probs else "log-linear E4M3 code"})},
        "forward_ms": round(ms_fwd, 4),
        "forward_tflops": round(fwd_tflops, 2),
        "forward_pct_fp8_peak": round(100.0 * fwd_tflops / FP8_PEAK_TFLOPS, 2),
        "quantize_ms": round(ms_quant, 4),
        "forward_protocol": fwd_proto,
        "forward_protocol_tflops": round(flops / (fwd_proto["median_ms"] * 1e-3) / 1e12, 2),
        "forward_protocol_pct_fp8_peak": round(100.0 * flops / (fwd_proto["median_ms"] * 1e-3) / 1e12
                                               / FP8_PEAK_TFLOPS, 2),
        "sclk_during_forward": sclk,
        "quantize_protocol": quant_proto,
        "step_protocol": step_proto,
        "mfma_skeleton": skeleton,
        "mfma_skeleton_random_operands": skeleton_random,
        "forward_frac_of_skeleton": round(fwd_tflops / skeleton["tflops"], 4) if skeleton else None,
        "forward_frac_of_random_skeleton": (round(fwd_tflops / skeleton_random["tflops"], 4)
                                            if skeleton_random else None),
        "roofline": {
            "kernel": "k_attn_mx (fp8attn_forward, FP4 plan)" if mx else "k_attn (fp8attn_forward)",
            "bound": "mfma",
            "achieved": round(fwd_tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(fwd_tflops / peak, 4),
            "traffic": traffic,
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            # codes: 1 B per element (E4M3) or 0.5 B + 1/32 B of scales (FP4) for Q, K, V; BF16 output
            "algorithmic_bytes": (int(3 * w.tokens * w.heads * (64 + 4) + 2 * w.tokens * w.heads * 128) if mx
                                  else 5 * w.tokens * w.heads * w.head_dim),
            # K/V streamed once per (XCD, round of its concurrent workgroups,
            # segment-head), Q once per item, output once: what per-XCD L2s allow
            "l2_stream_bytes": l2_floor,
        },
    }
    if args.copy_calibration > 0:
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = args.copy_calibration
        del src, dst
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
