#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

One step is one attn_fwd launch over the whole workload (inputs resident in
device memory). Prints ONE JSON line with throughput (TFLOP/s), the kernel's
roofline position against the dense fp16 MFMA peak, and the CPU oracle timed
on the host as a baseline (which also checks the GPU answer).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--prewarm-ms MS] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

# Published MI355X dense peaks / bandwidth (no sparsity).
PEAK_FP16_MFMA_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
PEAK_SCLK_MHZ = 2400.0  # the shader clock the MFMA peak is quoted at
# Exponential throughput used for the secondary (transcendental) bound: one
# v_exp_f32 per visible score; a wave64 v_exp_f32 issues every 9 cycles per
# SIMD (measured), 1024 SIMDs, at the 2.4 GHz peak clock.
EXP_PER_S = 1024 * 64 / 9.0 * 2.4e9
METRIC = "attn fwd TFLOP/s & µs, fp16 B1 H8 S4096 D64; % of dense FP16 MFMA peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prewarm-ms", type=float, default=250.0,
                    help="before the warmup steps, run the step back to back for this long "
                         "so that the GPU clock reaches its sustained level (0: off); "
                         "sweep and split-KV points get up to 100 ms each")
    ap.add_argument("--workload", default=None, help="workload name (default: the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle leg (for profiler runs)")
    ap.add_argument("--cpu-sample-rows", type=int, default=0,
                    help="rows per head for the CPU leg (0 = every row)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (HBM counter calibration)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the five-configuration timings, the sequence-length sweep "
                         "(4k/8k/16k, B1 H8 D64), the split-KV comparison, the kernel "
                         "variants and the key/value-cache (decode) timings")
    ap.add_argument("--sweep-steps", type=int, default=30,
                    help="timed launches per sweep point")
    ap.add_argument("--clock-seconds", type=float, default=1.0,
                    help="after the timed steps, run the step back to back this long while "
                         "rocm-smi samples the shader clock (0: skip)")
    ap.add_argument("--gemm-seconds", type=float, default=1.0,
                    help="time a plain fp16 library GEMM (8192^3, torch.matmul) back to back "
                         "this long as a reference for the dense MFMA rate this box sustains "
                         "(0: skip)")
    ap.add_argument("--cold", action="store_true",
                    help="also time launches with caches flushed (512 MB written before each)")
    ap.add_argument("--decode", default=None, metavar="WORKLOAD",
                    help="time only this key/value-cache (decode) workload and print its "
                         "record (for profiler runs)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("attn_fwd_kernel.h", "work_order.h", "plan.h", "attn_fwd.hip")


def kernel_label(w) -> str:
    """Name of the attention kernel instantiation a single pass of workload w
    launches (as rocprofv3 lists it): D = 64 runs three waves per SIMD
    (variant 128) from 2048 keys, causal folded pairs from 8192 keys. A label
    for the JSON line only; the library makes the choice."""
    var = 0
    if w.D == 64 and w.S >= 2048:
        nq = (w.S + 127) // 128
        folded = w.causal and w.B * w.H * ((nq + 1) // 2) >= 256
        if not w.causal or not folded or w.S >= 8192:
            var = 128
    return f"attn_fwd_kernel<{w.D},{str(w.causal).lower()},false,{var}>"


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and whitespace removed, so
    that a profile stays valid across comment-only edits."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_attention_forward_05_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def profiled_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this
    workload (FETCH_SIZE and WRITE_SIZE scaled by a plain-copy calibration), or
    None when there is none or the kernel source changed since it was taken."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    cur = kernel_source_hash()
    for name in sorted(os.listdir(pdir)):
        if not name.endswith(".md"):
            continue
        text = open(os.path.join(pdir, name)).read()
        for block in re.findall(r"```json\n(.*?)\n```", text, flags=re.S):
            try:
                rec = json.loads(block)
            except ValueError:
                continue
            if rec.get("workload") == workload and rec.get("source_hash") == cur:
                return rec.get("traffic_bytes_per_launch")
    return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def visible_scores(w) -> int:
    """Score elements the method exponentiates: S^2 per head, or S(S+1)/2 causal."""
    per_head = w.S * (w.S + 1) // 2 if w.causal else w.S * w.S
    return w.B * w.H * per_head


def cpu_baseline(w, q, k, v, o_gpu, lse_gpu, sample_rows: int):
    """Time the fp64 oracle on the host over a bounded sample of the workload and
    compare the GPU output with it on that sample."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()
                            if p.get("user_api") == "blas"] or [1])
    except Exception:
        blas_threads = 1
    S = w.S
    if sample_rows and sample_rows < S:
        rows = np.linspace(0, S - 1, sample_rows).round().astype(np.int64)
        desc = f"{sample_rows} evenly spaced query rows of each of the {w.B * w.H} heads"
    else:
        rows = None
        desc = f"the whole workload: all {w.B * w.H} heads x {S} query rows"
    t0 = time.perf_counter()
    if rows is None:
        O, L = oracle.sdpa_forward(q, k, v, w.scale, w.causal)
        n_rows = w.B * w.H * S
    else:
        O = np.empty((w.B, w.H, len(rows), w.D))
        L = np.empty((w.B, w.H, len(rows)))
        for b in range(w.B):
            for h in range(w.H):
                O[b, h], L[b, h] = oracle.sdpa_rows(q, k, v, w.scale, w.causal, b, h, rows)
        n_rows = w.B * w.H * len(rows)
    secs = time.perf_counter() - t0
    # FLOPs of the sample under the same convention as the GPU figure
    flops = w.flops * n_rows / (w.B * w.H * S)
    og = o_gpu if rows is None else o_gpu[:, :, rows]
    lg = lse_gpu if rows is None else lse_gpu[:, :, rows]
    err = np.abs(og.astype(np.float64) - O)
    parity = {"o_max_abs": float(err.max()), "o_mean_abs": float(err.mean()),
              "lse_max_abs": float(np.abs(lg.astype(np.float64) - L).max()),
              "pass": bool(err.max() <= 4e-3 and err.mean() <= 5e-4
                           and np.abs(lg.astype(np.float64) - L).max() <= 1e-3)}
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": blas_threads,
            "kind": "oracle", "sample": desc, "seconds": secs, "cpu_model": cpu_model(),
            "host_threads": os.cpu_count(),
            "note": "fp64 numpy oracle; matmuls on BLAS threads, exp/max/sum single-threaded"}, parity


def raw_step(entry, q, k, v, o, lse, w, stream, extra=()):
    """A launch of a C entry point with cached arguments (the checked Python
    binding has already accepted the same arguments once): keeps host
    overhead per launch well below the kernel time."""
    from exact_attention_forward_05_amd import _lib

    fn = getattr(_lib.load(), entry)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            w.B, w.H, w.S, w.D, w.scale, int(w.causal)) + tuple(extra) + (stream.cuda_stream,)

    def step():
        rc = fn(*args)
        if rc:
            _lib.check(rc)
    return step


LAUNCH_GROUP = 4  # launches between two events


def prewarm(step, ms):
    """Run ``step`` back to back for at least ``ms`` milliseconds of wall time
    (batches of 16, one synchronisation per batch). The MI355X shader clock
    ramps over tens of milliseconds of sustained load: without this the first
    few hundred launches of a run are up to 20% slower than the sustained
    rate. Returns {"ms": elapsed, "steps": launches}."""
    import torch

    n = 0
    t0 = time.perf_counter()
    while ms > 0 and (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(16):
            step()
        n += 16
        torch.cuda.synchronize()
    return {"ms": round((time.perf_counter() - t0) * 1e3, 1), "steps": n}


SCLK_RE = re.compile(r"GPU\[(\d+)\].*sclk clock level: \d+: \((\d+)\s*Mhz\)", re.I)


def parse_sclk(text: str):
    """{gpu index: MHz} from `rocm-smi --showclocks` output."""
    return {int(m.group(1)): int(m.group(2)) for m in SCLK_RE.finditer(text)}


def sample_sclk(step, seconds: float):
    """Run ``step`` back to back for ``seconds`` while a thread samples the
    shader clock with rocm-smi (a child process). The MI355X holds its power
    limit under this load, so the sustained clock, not the 2.4 GHz of the
    peak figure, sets the ceiling of the achieved rate. None when rocm-smi
    is missing or lists no single GPU."""
    import shutil
    import subprocess
    import threading

    import torch

    exe = shutil.which("rocm-smi")
    if exe is None or seconds <= 0:
        return None
    samples, gpus = [], set()
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                r = subprocess.run([exe, "--showclocks"], capture_output=True, text=True, timeout=10)
                clk = parse_sclk(r.stdout)
                gpus.update(clk)
                if len(clk) == 1:
                    samples.append(next(iter(clk.values())))
            except (OSError, subprocess.SubprocessError):
                pass
            stop.wait(0.05)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    if not samples:
        return None
    # the first samples may still see the ramp; report the later half
    late = samples[len(samples) // 2:]
    return {"mhz_median": float(np.median(late)), "mhz_min": min(late), "mhz_max": max(late),
            "samples": len(late), "seconds": seconds}


def time_launches(step, stream, steps):
    """Launch ``step`` ``steps`` times back to back, with a pair of HIP events
    on the launch stream around every group of LAUNCH_GROUP launches (an event
    between every two kernels would add its own gap to each). Returns
    (per-launch ms of each group, wall seconds)."""
    import torch

    groups = max(1, steps // LAUNCH_GROUP)
    sizes = [LAUNCH_GROUP] * groups
    sizes[-1] += steps - LAUNCH_GROUP * groups
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(groups)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(groups)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, n in enumerate(sizes):
        starts[i].record(stream)
        for _ in range(n):
            step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return np.array([s.elapsed_time(e) / n for s, e, n in zip(starts, ends, sizes)]), wall


def time_cold(step, dev, stream, steps):
    """Per-launch time with the L2 and the infinity cache flushed: a 512 MB
    buffer is written on the same stream before each launch, outside the
    event pair around it."""
    import torch

    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    durs = []
    for _ in range(steps):
        scratch.fill_(1)
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        step()
        s1.record(stream)
        durs.append((s0, s1))
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in durs])
    del scratch
    return {"us_mean": round(float(ms.mean()) * 1e3, 3),
            "us_median": round(float(np.median(ms)) * 1e3, 3), "launches": steps}


def time_workload(attn, dev, stream, name, steps, prewarm_ms):
    """Kernel time of one workload: pre-warm, 5 launches, then `steps` timed
    launches in event-bracketed groups. Returns the record for the JSON line."""
    import torch

    from testkit import WORKLOADS, workload_inputs

    w = WORKLOADS[name]
    q, k, v = (torch.from_numpy(x).to(dev) for x in workload_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)

    attn.fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse, stream=stream)
    step = raw_step("attn_fwd", q, k, v, o, lse, w, stream)
    prewarm(step, prewarm_ms)
    for _ in range(5):
        step()
    durs, _ = time_launches(step, stream, steps)
    mean_ms = float(durs.mean())
    rec = {"workload": name, "B": w.B, "H": w.H, "S": w.S, "D": w.D, "causal": w.causal,
           "us_mean": round(mean_ms * 1e3, 3),
           "us_median": round(float(np.median(durs)) * 1e3, 3),
           "tflops": round(w.flops / (mean_ms * 1e-3) / 1e12, 2),
           "pct_of_peak": round(100 * w.flops / (mean_ms * 1e-3) / 1e12
                                / PEAK_FP16_MFMA_TFLOPS, 2)}
    del q, k, v, o, lse
    return rec


def run_sweep(attn, dev, stream, steps, prewarm_ms):
    """Kernel time over the sequence-length sweep (B1 H8 D64; S = 4k, 8k, 16k;
    non-causal and causal)."""
    from testkit import SWEEP

    out = []
    for (S, causal), name in sorted(SWEEP.items(), key=lambda kv: (kv[0][1], kv[0][0])):
        rec = time_workload(attn, dev, stream, name, steps, prewarm_ms)
        out.append({"workload": name, "S": S, "causal": causal,
                    **{k: rec[k] for k in ("us_mean", "us_median", "tflops", "pct_of_peak")}})
        log(f"sweep {name}: {out[-1]['us_mean']} us, {out[-1]['tflops']} TFLOP/s")
    return out


def run_configs(attn, dev, stream, steps, prewarm_ms):
    """Kernel time of each of the five problem configurations."""
    from testkit import CONFIGS

    out = []
    for name in CONFIGS:
        out.append(time_workload(attn, dev, stream, name, steps, prewarm_ms))
        log(f"config {name}: {out[-1]['us_mean']} us, {out[-1]['tflops']} TFLOP/s")
    return out


def run_splitkv(attn, dev, stream, steps, prewarm_ms):
    """Single-pass vs split-KV (split count from the library's heuristic) on
    workloads that leave CUs idle or unbalanced in one pass."""
    import torch

    from testkit import SPLITKV_BENCH, WORKLOADS, workload_inputs

    out = []
    for name in SPLITKV_BENCH:
        w = WORKLOADS[name]
        q, k, v = (torch.from_numpy(x).to(dev) for x in workload_inputs(w))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
        ns = attn.choose_splits(w.B, w.H, w.S, w.D, w.causal,
                                torch.cuda.get_device_properties(dev).multi_processor_count)
        ws = torch.empty(max(1, attn.splitkv_workspace_size(w.B, w.H, w.S, w.D, ns)),
                         dtype=torch.uint8, device=dev)

        attn.fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse, stream=stream)
        attn.fwd_splitkv(q, k, v, n_splits=ns, scale=w.scale, causal=w.causal, out=o,
                         lse=lse, workspace=ws, stream=stream)
        single = raw_step("attn_fwd", q, k, v, o, lse, w, stream)
        split = raw_step("attn_fwd_splitkv", q, k, v, o, lse, w, stream,
                         extra=(ns, ws.data_ptr(), ws.numel()))

        # three interleaved rounds (as for the variants): per tag, the round
        # means and medians, reported as their medians
        rec = {"workload": name, "n_splits": ns, "rounds": 3}
        runs = {"single_pass": ([], []), "splitkv": ([], [])}
        for _ in range(3):
            for tag, fn in (("single_pass", single), ("splitkv", split)):
                prewarm(fn, prewarm_ms)
                for _ in range(5):
                    fn()
                durs, _ = time_launches(fn, stream, steps)
                runs[tag][0].append(float(durs.mean()) * 1e3)
                runs[tag][1].append(float(np.median(durs)) * 1e3)
        for tag, (means, medians) in runs.items():
            mean_us = float(np.median(means))
            rec[f"{tag}_us_mean"] = round(mean_us, 3)
            rec[f"{tag}_us_median"] = round(float(np.median(medians)), 3)
            rec[f"{tag}_tflops"] = round(w.flops / (mean_us * 1e-6) / 1e12, 2)
        rec["speedup"] = round(rec["single_pass_us_mean"] / rec["splitkv_us_mean"], 3)
        log(f"splitkv {name}: {rec}")
        out.append(rec)
        del q, k, v, o, lse, ws
    return out


# Kernel variants timed against the default kernel: (workload, variant).
VARIANT_BENCH = (("sdpa_b1h8s4096d64", 1), ("sdpa_b1h8s4096d64", 2), ("sdpa_b1h8s4096d64", 4),
                 ("sdpa_b1h8s4096d64", 8), ("sdpa_b1h8s4096d64", 32),
                 ("long_b1h8s16384d64", 1), ("long_b1h8s16384d64", 2),
                 ("long_b1h8s16384d64", 4), ("long_b1h8s16384d64", 8),
                 ("long_b1h8s16384d64", 32), ("sdpa_b1h8s4096d64", 64),
                 ("long_b1h8s16384d64", 64), ("sdpa_b1h8s4096d64", 256),
                 ("sdpa_b1h8s4096d64", 512), ("long_b1h8s16384d64", 512),
                 ("sdpa_b1h8s4096d64", 1152), ("long_b1h8s16384d64", 1152),
                 ("causal_b2h16s8192d128", 2))
VARIANT_NAMES = {1: "ring3", 2: "exp_poly", 4: "wide", 8: "subpipe", 32: "bar2", 64: "prod",
                 128: "trio", 256: "quad", 512: "rot", 1024: "m32", 1152: "m32_trio"}


def run_variants(attn, dev, stream, steps, prewarm_ms, rounds: int = 3):
    """Kernel time of each compiled variant against the default kernel on the
    same inputs (attn_fwd_variant): ``rounds`` rounds, each timing the default
    and then every variant, each pre-warmed; medians over the rounds, so that
    a drift of the power-limited clock during the section does not favour
    whichever build runs in a given place of the order."""
    import torch

    from testkit import WORKLOADS, workload_inputs

    out = []
    by_wl = {}
    for name, var in VARIANT_BENCH:
        by_wl.setdefault(name, []).append(var)
    for name, variants in by_wl.items():
        w = WORKLOADS[name]
        q, k, v = (torch.from_numpy(x).to(dev) for x in workload_inputs(w))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)

        def timed(fn):
            prewarm(fn, prewarm_ms)
            for _ in range(5):
                fn()
            durs, _ = time_launches(fn, stream, steps)
            return float(durs.mean()) * 1e3

        # every build once through the checked binding, then raw launches
        attn.fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse, stream=stream)
        for var in variants:
            attn.fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse, stream=stream,
                     variant=var)
        steps_of = {0: raw_step("attn_fwd", q, k, v, o, lse, w, stream)}
        for var in variants:
            steps_of[var] = raw_step("attn_fwd_variant", q, k, v, o, lse, w, stream, extra=(var,))
        times = {key: [] for key in steps_of}
        for _ in range(rounds):
            for key, fn in steps_of.items():
                times[key].append(timed(fn))
        base_us = float(np.median(times[0]))
        for var in variants:
            us = float(np.median(times[var]))
            rec = {"workload": name, "variant": VARIANT_NAMES[var], "default_us": round(base_us, 3),
                   "variant_us": round(us, 3), "variant_tflops": round(w.flops / (us * 1e-6) / 1e12, 2),
                   "ratio": round(us / base_us, 4), "rounds": rounds}
            log(f"variant {rec}")
            out.append(rec)
        del q, k, v, o, lse
    return out


def run_decode(attn, dev, stream, steps, prewarm_ms, names=None):
    """Queries against a key/value cache (attn_fwd_kvcache, split count from
    the library's model): kernel time of the split pass plus the combine,
    against the HBM roofline (K and V read once dominate the bytes)."""
    import torch

    from exact_attention_forward_05_amd import _lib
    from testkit import DECODE, cache_inputs

    out = []
    for name, w in DECODE.items():
        if names is not None and name not in names:
            continue
        q, k, v = (torch.from_numpy(x).to(dev) for x in cache_inputs(w))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device=dev)
        ns = attn.choose_splits(w.B, w.H, w.Sq, w.D, w.causal,
                                torch.cuda.get_device_properties(dev).multi_processor_count,
                                Sk=w.Sk)
        ws = torch.empty(max(16, attn.splitkv_workspace_size(w.B, w.H, w.Sq, w.D, ns)),
                         dtype=torch.uint8, device=dev)
        attn.fwd_kvcache(q, k, v, n_splits=ns, scale=w.scale, causal=w.causal, out=o, lse=lse,
                         workspace=ws, stream=stream)
        fn = getattr(_lib.load(), "attn_fwd_kvcache")
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.H,
                w.Sq, w.Sk, w.D, w.scale, int(w.causal), ns, ws.data_ptr(), ws.numel(),
                stream.cuda_stream)

        def step():
            rc = fn(*args)
            if rc:
                _lib.check(rc)
        prewarm(step, prewarm_ms)
        for _ in range(5):
            step()
        durs, _ = time_launches(step, stream, steps)
        us = float(durs.mean()) * 1e3
        # partial results written and read back by the combine (fp32 o/d and lse)
        part = 2 * ns * w.B * w.H * w.Sq * (w.D + 1) * 4 if ns > 1 else 0
        rec = {"workload": name, "B": w.B, "H": w.H, "S_q": w.Sq, "S_k": w.Sk, "D": w.D,
               "causal": w.causal, "n_splits": ns, "us_mean": round(us, 3),
               "algorithmic_bytes": w.algorithmic_bytes, "partial_bytes": part,
               "hbm_gbs": round(w.algorithmic_bytes / (us * 1e-6) / 1e9, 1),
               "hbm_frac": round(w.algorithmic_bytes / (us * 1e-6) / (PEAK_HBM_GBS * 1e9), 4),
               "tflops": round(w.flops / (us * 1e-6) / 1e12, 2)}
        log(f"decode {rec}")
        out.append(rec)
        del q, k, v, o, lse, ws
    return out


def gemm_reference(dev, seconds: float, n: int = 8192):
    """Sustained rate of a plain fp16 GEMM from the vendor library
    (torch.matmul -> hipBLASLt, fp32 accumulation) on this machine: a reference
    for the dense MFMA rate a tuned contraction reaches at the power-limited
    clock, beside the published peak. Not part of the attention path."""
    import torch

    if seconds <= 0:
        return None
    try:
        g = torch.Generator(device=dev).manual_seed(7)
        a = torch.randn(n, n, device=dev, generator=g).half()
        b = torch.randn(n, n, device=dev, generator=g).half()
        c = torch.empty(n, n, dtype=torch.float16, device=dev)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        rates = []
        while time.perf_counter() - t0 < seconds:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(4):
                torch.matmul(a, b, out=c)
            e1.record()
            torch.cuda.synchronize(dev)
            rates.append(4 * 2.0 * n ** 3 / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        del a, b, c
    except RuntimeError as e:  # e.g. out of memory: the reference is optional
        log(f"fp16 GEMM reference skipped: {e}")
        return None
    late = rates[len(rates) // 2:]
    return {"tflops": round(float(np.median(late)), 1), "m_n_k": [n, n, n], "dtype": "f16",
            "library": "torch.matmul (hipBLASLt)", "seconds": seconds}


def copy_calibration(dev):
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE per dispatch
    calibrate the HBM byte counters read for the attention kernels."""
    import torch

    nbytes = 256 << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    log(f"copy calibration: 3 copies of {nbytes} bytes")
    del src, dst


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py is single-GPU; launch it without torch.distributed", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_attention_forward_05_amd as attn
    from testkit import DECODE, HEADLINE, WORKLOADS, workload_inputs

    dev = torch.device("cuda:0")
    if args.decode is not None:
        if args.decode not in DECODE:
            print(json.dumps({"error": f"unknown decode workload {args.decode}",
                              "choices": sorted(DECODE)}))
            sys.exit(2)
        recs = run_decode(attn, dev, torch.cuda.current_stream(dev), args.steps,
                          args.prewarm_ms, names=(args.decode,))
        if args.copy_calibration:  # after the inputs' host-to-device copies
            copy_calibration(dev)
        print(json.dumps({"decode": recs[0]}))
        return
    w = WORKLOADS[args.workload or HEADLINE]
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")
    log(f"workload {w.name}: {w.describe()}")
    q, k, v = workload_inputs(w)
    qt, kt, vt = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    o = torch.empty_like(qt)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    # The first call goes through the checked binding; the timed loop then
    # calls the C entry point with the same (cached) arguments, so that host
    # overhead per launch stays below the kernel time.
    attn.fwd(qt, kt, vt, scale=w.scale, causal=w.causal, out=o, lse=lse, stream=stream)
    step = raw_step("attn_fwd", qt, kt, vt, o, lse, w, stream)

    if args.copy_calibration:
        copy_calibration(dev)

    pre = prewarm(step, args.prewarm_ms)
    log(f"prewarm: {pre['steps']} launches in {pre['ms']} ms")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    log(f"warmup {args.warmup} done")

    # Per-launch device time from events recorded on the launch stream.
    durs_ms, wall = time_launches(step, stream, args.steps)
    avg_ms = float(durs_ms.mean())
    log(f"timed {args.steps} steps: wall {wall * 1e3:.2f} ms, per launch (groups of "
        f"{LAUNCH_GROUP}) avg {avg_ms * 1e3:.2f} us, median {np.median(durs_ms) * 1e3:.2f} us, "
        f"min {durs_ms.min() * 1e3:.2f} us")

    sclk = sample_sclk(step, args.clock_seconds)
    log(f"shader clock under sustained launches: {sclk}")
    gemm = gemm_reference(dev, args.gemm_seconds)
    log(f"fp16 library GEMM reference: {gemm}")

    ms_per_step = wall * 1e3 / args.steps
    value = w.flops / (ms_per_step * 1e-3) / 1e12
    achieved = w.flops / (avg_ms * 1e-3) / 1e12
    traffic = profiled_traffic(w.name)
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm": pre,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S": w.S, "D": w.D,
                   "causal": w.causal, "scale": w.scale, "seed": w.seed,
                   "qk_mult": w.qk_mult},
        "us_per_launch": {"mean": round(avg_ms * 1e3, 3),
                          "median": round(float(np.median(durs_ms)) * 1e3, 3),
                          "min": round(float(durs_ms.min()) * 1e3, 3)},
        "pct_of_peak": round(100.0 * achieved / PEAK_FP16_MFMA_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3),
                     "peak": PEAK_FP16_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP16_MFMA_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": kernel_label(w),
                     # the shader clock sampled under the same launches, and the
                     # fraction of the peak scaled to that clock (informative)
                     "sclk_mhz": None if sclk is None else sclk["mhz_median"],
                     # the rate a plain fp16 library GEMM sustains on the same box
                     "gemm_reference_tflops": None if gemm is None else gemm["tflops"],
                     "frac_of_gemm": (None if gemm is None
                                      else round(achieved / gemm["tflops"], 4)),
                     "frac_at_sclk": (None if sclk is None else round(
                         achieved / (PEAK_FP16_MFMA_TFLOPS * sclk["mhz_median"] / PEAK_SCLK_MHZ), 4)),
                     "algorithmic_flops_per_launch": w.flops,
                     "algorithmic_bytes_per_launch": w.algorithmic_bytes},
        # secondary bounds at the same launch time: exponentials and HBM
        "exp_bound": {"exps_per_launch": visible_scores(w),
                      "us_at_exp_peak": round(visible_scores(w) / EXP_PER_S * 1e6, 3),
                      "frac": round(visible_scores(w) / EXP_PER_S / (avg_ms * 1e-3), 4)},
        "hbm_bound": {"us_at_hbm_peak": round(w.algorithmic_bytes / (PEAK_HBM_GBS * 1e9) * 1e6, 3),
                      "frac": round(w.algorithmic_bytes / (avg_ms * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
                      # GB/s of the algorithmic bytes, and of the profiled HBM traffic
                      "algorithmic_gbs": round(w.algorithmic_bytes / (avg_ms * 1e-3) / 1e9, 1),
                      "traffic_gbs": (None if traffic is None
                                      else round(traffic / (avg_ms * 1e-3) / 1e9, 1))},
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count},
    }
    if args.cold:
        result["cold"] = time_cold(step, dev, stream, min(args.steps, 50))
        log(f"cold launches: {result['cold']}")
    if not args.no_sweep:
        point_ms = min(args.prewarm_ms, 100.0)
        result["configs"] = run_configs(attn, dev, stream, args.sweep_steps, point_ms)
        result["sweep"] = run_sweep(attn, dev, stream, args.sweep_steps, point_ms)
        result["splitkv"] = run_splitkv(attn, dev, stream, args.sweep_steps, point_ms)
        result["variants"] = run_variants(attn, dev, stream, args.sweep_steps, point_ms)
        result["decode"] = run_decode(attn, dev, stream, args.sweep_steps, point_ms)
    if not args.no_cpu_baseline:
        log("CPU oracle leg ...")
        o_np = o.cpu().numpy()
        l_np = lse.cpu().numpy()
        base, parity = cpu_baseline(w, q, k, v, o_np, l_np, args.cpu_sample_rows)
        result["cpu_baseline"] = base
        result["parity"] = parity
        log(f"CPU oracle {base['seconds']:.2f} s, parity {parity}")
        if not parity["pass"]:
            log("PARITY FAILED: the GPU result does not match the oracle")
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    if result.get("parity") and not result["parity"]["pass"]:
        sys.exit(1)


if __name__ == "__main__":
    main()
