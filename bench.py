#!/usr/bin/env python3
"""Benchmark of the exact attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long] [--legs LIST]

Prints ONE JSON line on stdout (progress goes to stderr).  A step is one call
of the attention forward over one batch of the workload.  The headline
workload is the long-context causal prefill (B=1, H=12, T=16384, d=64, bf16):
the largest prefill configuration, on which the prefill kernel runs every
step of the hot path (Q tile load, K/V streaming, both products, the online
softmax, causal skipping, the epilogue).

Every other configuration is a leg of the same line, measured the same way
(LEGS below): the GPT-2-shaped prefill (4x12x1024, causal), the mid-length
prefill non-causal and causal (2x16x4096, K x 3), the mid-length prefill at
head width 128, the backward pass, a 16K-token single-head prefill with the
key axis split across workgroups, the split-KV decode step (64x32, 8192 keys,
d=128, 16 partitions), its grouped-query form and a batch-1 decode step.

Per leg: K timed steps (HIP events on the stream the kernels are launched on,
bracketed by device synchronisation; for a leg whose K calls last under
10 ms, as many calls as fill 10 ms, the count in its "steps") after a
clock-settling phase of back-to-back calls and W untimed warm-up steps
(the headline always times exactly K steps); three repeats of at least
50 ms of back-to-back calls (per-call median and spread); the roofline
fraction against the vendor peak, with the HBM bytes of committed rocprofv3
counter summaries when they were taken on the current kernel sources; parity
against the float64 oracle on whole heads or sampled rows of the same GPU
output; the oracle timed on the host cores on a bounded sample; and the peak
device memory a call needs beyond its inputs, measured (caching-allocator
peak around a call that allocates its own outputs and workspace, and the
device's free memory around a call on preallocated buffers).
Inputs are seeded synthetic tensors already resident in HBM when timing
starts.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PEAK_F32_VALU_TFLOPS = 157.3  # MI355X fp32 vector (256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2 (packed) x 2.4 GHz)
PROFILES = os.path.join(ROOT, "profiles")

HEADLINE = "long"
# legs of the line, in the order they run
LEGS = ("gpt2", "mid", "mid_causal", "mid_d128", "backward", "prefill_split", "decode", "decode_gqa", "decode_b1")
PREFILL_LEGS = ("gpt2", "mid", "mid_causal", "mid_d128")
DECODE_LEGS = ("decode", "decode_gqa", "decode_b1")

# "Attention and Its Computational Cost", section "What the causal mask saves":
# causal time over full time of the memory-efficient kernel at T = 1024 / 2048
# / 4096 (the work ratio is 0.5)
PAGES_CAUSAL_RATIO = {"efficient": [0.71, 0.59, 0.58], "work_ratio": 0.5}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_pairs(tq: int, tkv: int, causal: bool) -> int:
    """(query, key) pairs attention touches; causal uses bottom-right alignment."""
    if not causal:
        return tq * tkv
    off = tkv - tq
    return tq * (off + 1) + tq * (tq - 1) // 2


def prefill_flops(w) -> int:
    return 4 * w.B * w.H * w.d * visible_pairs(w.Tq, w.Tkv, w.causal)


def prefill_bytes(w) -> int:
    es = 2 if w.dtype == "bf16" else 4
    return w.B * w.H * ((2 * w.Tq + 2 * w.Tkv) * w.d * es + w.Tq * 4)


def prefill_output_bytes(w) -> int:
    """O (same dtype as q) and the fp32 LSE."""
    es = 2 if w.dtype == "bf16" else 4
    return w.B * w.H * w.Tq * (w.d * es + 4)


def decode_bytes(w) -> tuple[int, int]:
    """(all bytes, K/V-cache bytes) one decode step must move: K and V once
    (kv_heads of them), q in, O and LSE out."""
    kv = 2 * w.B * w.kv_heads * w.Tkv * w.d * 2
    return kv + 2 * w.B * w.H * w.d * 2 + w.B * w.H * 4, kv


def prefill_roofline(w, ms: float) -> dict:
    """The bound of a prefill launch (whichever of the algorithmic bytes at
    the HBM peak and the flops at the compute peak takes longer) and the
    fraction of that peak the measured time reaches."""
    flops, nbytes = prefill_flops(w), prefill_bytes(w)
    # bf16 products run on the matrix cores; the fp32 path's are VALU FMAs
    peak, bound = (PEAK_BF16_TFLOPS, "mfma") if w.dtype == "bf16" else (PEAK_F32_VALU_TFLOPS, "alu")
    if nbytes / (PEAK_HBM_GBPS * 1e9) > flops / (peak * 1e12):
        ach = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBPS}
    tf = flops / (ms * 1e-3) / 1e12
    return {"bound": bound, "achieved": tf, "peak": peak, "unit": "TFLOP/s", "frac": tf / peak}


def kernel_sources_digest() -> str:
    """Digest of the device sources (the kernels, their launch rules and the
    headers they share: every .hip and .hpp file) with comments and whitespace
    removed, so that only a change to kernel code invalidates recorded
    counters.  The host-side argument checks (.cpp) run before any launch and
    do not enter it; which kernel a call reaches is checked by name."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "io_aware_exact_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if not f.endswith((".hip", ".hpp")):
            continue
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(f.encode() + b"\0" + text.encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel_prefix: str, workload: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, only if
    they were taken on the current device sources and on the kernel that ran
    (`kernel`, as attn_last_kernel names it); otherwise None."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        e = rec.get(workload, {}).get(kernel_prefix)
        if not e or e.get("sources_sha256_16") != kernel_sources_digest() or e.get("kernel") != kernel:
            return None
        return int(e["fetch_bytes"] + e["write_bytes"])
    except (OSError, ValueError, KeyError, TypeError):
        return None


def parse_rocminfo_clock(text: str):
    """Max clock (MHz) of the first gfx950 agent in `rocminfo` output."""
    agent = None
    for line in text.splitlines():
        s = line.strip()
        if s.startswith("Name:"):
            agent = s.split(":", 1)[1].strip()
        elif s.startswith("Max Clock Freq. (MHz):") and agent and agent.startswith("gfx950"):
            try:
                return int(s.split(":", 1)[1].strip())
            except ValueError:
                return None
    return None


def device_max_clock_mhz():
    try:
        r = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60)
        return parse_rocminfo_clock(r.stdout)
    except (OSError, subprocess.SubprocessError):
        return None


# ------------------------------------------------------------------ timing

def settle(torch, call, settle_ms: float) -> float:
    """Back-to-back calls for about settle_ms of device time, so the timed
    steps start at the clock the chip holds under this load rather than on
    its ramp; returns the milliseconds spent."""
    if settle_ms <= 0:
        return 0.0
    t0 = time.perf_counter()
    for _ in range(4):
        call()
    torch.cuda.synchronize()
    per = max((time.perf_counter() - t0) / 4, 1e-6)
    for _ in range(min(200000, math.ceil(settle_ms * 1e-3 / per))):
        call()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3


def time_steps(torch, call, steps: int, warmup: int):
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        call()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_leg(torch, call, steps: int, warmup: int, min_ms: float = 10.0):
    """A leg's timed steps: the requested K steps, or, when K calls take less
    than min_ms (where one late launch moves the mean), as many back-to-back
    calls as fill min_ms.  Returns (ms per call, calls timed).  The headline
    always times exactly K steps."""
    ms = time_steps(torch, call, steps, warmup)
    if ms * steps >= min_ms:
        return ms, steps
    n = math.ceil(min_ms / max(ms, 1e-4))
    return time_steps(torch, call, n, 1), n


def time_repeats(torch, call, ms_per_call: float, reps: int = 3, min_ms: float = 50.0):
    """Repeats of N back-to-back calls, N chosen so that each repeat lasts at
    least min_ms: the per-call time of each repeat, their median and spread
    (max - min), beside the K-step number."""
    n = max(1, math.ceil(min_ms / max(ms_per_call, 1e-4)))
    ts = sorted(time_steps(torch, call, n, 1) for _ in range(reps))
    return {"calls_per_repeat": n, "ms_per_call": ts, "median_ms": ts[len(ts) // 2], "spread_ms": ts[-1] - ts[0]}


def time_cold(torch, call, reps: int = 30):
    """Median per-call time with a 512 MiB write between calls, which evicts
    the L2 caches and the 256 MiB last-level cache, so every call starts with
    its inputs in HBM only (HIP events on the launch stream around each call)."""
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    call()
    ts = []
    for i in range(reps):
        scrub.fill_(i & 0xFF)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        call()
        end.record()
        torch.cuda.synchronize()
        ts.append(start.elapsed_time(end))
    del scrub
    ts.sort()
    return ts[len(ts) // 2], ts[0], ts[-1]


def measure_memory(torch, prepared_call, alloc_call, input_bytes: int, output_bytes: int,
                   workspace_bytes: int = 0) -> dict:
    """Device memory a call needs beyond its inputs, measured two ways.

    * The device's free memory before and after a call on preallocated
      buffers (the library itself allocates nothing; any growth shows here).
    * The caching allocator's peak around a binding call that allocates its
      own outputs and workspace: the peak above the memory held before the
      call is outputs + workspace + anything else the call needed.

    ``extra_device_bytes`` = that peak minus the outputs the call returns,
    plus any free-memory drop: the memory beyond inputs and outputs.
    ``peak_beyond_inputs_bytes`` = the allocator peak (outputs included), the
    quantity of the pages' peak-extra-memory table."""
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    prepared_call()
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    lib_delta = max(0, free0 - free1)
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    res = alloc_call()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    held = torch.cuda.memory_allocated() - base      # the returned outputs
    del res
    return {"extra_device_bytes": max(0, peak - held) + lib_delta,
            "peak_beyond_inputs_bytes": peak + lib_delta,
            "output_bytes_allocated": held, "output_bytes_algorithmic": output_bytes,
            "workspace_bytes": workspace_bytes, "library_free_memory_drop_bytes": lib_delta,
            "input_bytes": input_bytes,
            "method": "torch caching-allocator peak around a call that allocates its own outputs and workspace; "
                      "hipMemGetInfo free bytes around a call on preallocated buffers"}


# ------------------------------------------------------------------ oracle legs

def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def sampled_rows(T: int, n: int, rng):
    """First and last rows, rows around tile edges and a random spread."""
    import numpy as np
    edge = [0, 1, 31, 32, 63, 64, 127, 128, 129, T // 2, T - 129, T - 128, T - 2, T - 1]
    rnd = rng.choice(T, size=min(n, T), replace=False).tolist()
    return np.array(sorted(set(r for r in edge + rnd if 0 <= r < T)))


# per workload: heads checked and rows per head (None = every row)
PARITY_PLAN = {"gpt2": ("all", None), "mid": (3, None), "mid_causal": (3, None), "long": (2, 512),
               "mid_d128": (2, None), "tiny": ("all", None)}


def prefill_parity(w, q, k, v, o_gpu, lse_gpu) -> dict:
    """Max-abs errors of the GPU output against the float64 oracle on the
    heads and rows of PARITY_PLAN (the same GPU output that was timed)."""
    import numpy as np

    import oracle
    from io_aware_exact_amd.inputs import to_f64

    nheads, nrows = PARITY_PLAN.get(w.name, (2, 256))
    all_heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    rng = np.random.default_rng(4242 + w.seed)
    if nheads == "all":
        heads = all_heads
    else:
        heads = [all_heads[0], all_heads[-1]]
        extra = [all_heads[i] for i in rng.permutation(len(all_heads)) if all_heads[i] not in heads]
        heads += extra[:max(0, nheads - 2)]
    eo = el = 0.0
    checked = 0
    for b, h in heads:
        rows = None if nrows is None else sampled_rows(w.Tq, nrows, rng)
        o_ref, lse_ref = oracle.attention(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]), w.scale, w.causal,
                                          rows=rows)
        og, lg = o_gpu[b, h], lse_gpu[b, h]
        if rows is not None:
            og, lg = og[rows], lg[rows]
        eo = max(eo, float(np.abs(to_f64(og) - o_ref).max()))
        el = max(el, float(np.abs(to_f64(lg) - lse_ref).max()))
        checked += w.Tq if rows is None else rows.size
    tol = 1e-5 if w.dtype == "f32" else 2e-2
    return {"max_abs_err_o": eo, "max_abs_err_lse": el, "tol_o": tol, "tol_lse": 1e-3,
            "ok": bool(eo <= tol and el <= 1e-3), "heads_checked": len(heads), "rows_checked": checked,
            "rows_per_head": "all" if nrows is None else nrows}


def cpu_baseline_prefill(w, q, k, v, min_seconds: float) -> dict:
    """The float64 oracle on the host over whole (b, h) heads of the same
    inputs until about ``min_seconds`` of CPU work is done."""
    import oracle
    from io_aware_exact_amd.inputs import to_f64

    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, t_compute, t_convert = 0, 0.0, 0.0
    t_wall0 = time.perf_counter()
    while t_compute < min_seconds:
        b, h = heads[done % len(heads)]
        t0 = time.perf_counter()
        qb, kb, vb = to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h])
        t_convert += time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.attention(qb, kb, vb, w.scale, w.causal)
        t_compute += time.perf_counter() - t0
        done += 1
    per_head = 4 * w.d * visible_pairs(w.Tq, w.Tkv, w.causal)
    return {
        "value": per_head * done / t_compute / 1e12,
        "unit": "TFLOP/s",
        "cores": blas_threads(),
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{done} (batch, head) slices of this workload ({done / len(heads):.2f} x its {len(heads)} "
                  f"slices), float64 numpy, full T_q x T_kv scores materialised per head; causal-adjusted flop count",
        "seconds": t_compute,
        "conversion_seconds": t_convert,
        "wall_seconds": time.perf_counter() - t_wall0,
    }


# ------------------------------------------------------------------ legs

def workload_label(w, kind="prefill") -> str:
    return (f"{w.name} {kind} B={w.B} H={w.H} Tq={w.Tq} Tkv={w.Tkv} d={w.d} "
            f"{'causal' if w.causal else 'non-causal'} {w.dtype}")


def run_prefill(torch, attn, name, args, cpu_seconds: float, cold: bool = False, headline: bool = False) -> dict:
    """One prefill workload: timing, repeats, roofline, parity, oracle leg and
    memory, all on the same inputs."""
    from io_aware_exact_amd.inputs import WORKLOADS, make_qkv

    w = WORKLOADS[name]
    log(f"[bench] {name}: {w}")
    q, k, v = make_qkv(w)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty_like(dq)
    lse = torch.empty((w.B, w.H, w.Tq), dtype=torch.float32, device="cuda")
    f32 = w.dtype == "f32"
    call = attn.prepared_fwd(dq, dk, dv, o, lse, w.causal, w.scale, f32=f32)
    settled = settle(torch, call, args.settle_ms)
    if headline:
        ms, nsteps = time_steps(torch, call, args.steps, args.warmup), args.steps
    else:
        ms, nsteps = time_leg(torch, call, args.steps, args.warmup)
    kern = attn.attn_last_kernel()
    reps = time_repeats(torch, call, ms)
    flops = prefill_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    roof = prefill_roofline(w, ms)
    roof["traffic"] = measured_traffic("prefill", w.name, kern)
    log(f"[bench] {name} {kern}: {ms * 1e3:.2f} us/step, {tflops:.1f} TFLOP/s "
        f"(repeats median {reps['median_ms'] * 1e3:.2f} us)")
    fwd = attn.attn_fwd_f32 if f32 else attn.attn_fwd
    mem = measure_memory(torch, call, lambda: fwd(dq, dk, dv, causal=w.causal, scale=w.scale),
                         3 * dq.numel() * dq.element_size(), prefill_output_bytes(w))
    out = {
        "workload": workload_label(w),
        "metric": "attn fwd TFLOP/s (causal-adjusted)",
        "value": tflops,
        "unit": "TFLOP/s",
        "ms_per_step": ms,
        "steps": nsteps,
        "warmup": args.warmup,
        "settle_ms": settled,
        "kernel": kern,
        "flops_per_call": flops,
        "algorithmic_bytes_per_call": prefill_bytes(w),
        "pct_of_peak": {("bf16_mfma" if not f32 else "f32_valu"): 100.0 * tflops / (PEAK_F32_VALU_TFLOPS if f32 else PEAK_BF16_TFLOPS),
                        "hbm_algorithmic": 100.0 * prefill_bytes(w) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS},
        "roofline": roof,
        "repeats": reps,
        "memory": mem,
        "extra_device_bytes": mem["extra_device_bytes"],
    }
    if cold:
        cold_ms, cold_min, cold_max = time_cold(torch, call)
        out["cold_cache"] = {"ms_per_call": cold_ms, "min_ms": cold_min, "max_ms": cold_max,
                             "value": flops / (cold_ms * 1e-3) / 1e12, "unit": "TFLOP/s",
                             "protocol": "512 MiB write before each call, per-call HIP events, median of 30"}
        log(f"[bench] {name} with caches scrubbed between calls: {cold_ms * 1e3:.2f} us/call")
    o_host, lse_host = o.cpu(), lse.cpu()
    del dq, dk, dv, o, lse
    torch.cuda.empty_cache()
    out["parity"] = prefill_parity(w, q, k, v, o_host, lse_host)
    log(f"[bench] {name} parity {out['parity']}")
    if cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline_prefill(w, q, k, v, cpu_seconds)
        log(f"[bench] {name} oracle {out['cpu_baseline']['value']:.4f} TFLOP/s on "
            f"{out['cpu_baseline']['cores']} threads")
    else:
        out["cpu_baseline"] = None
    return out


def run_decode(torch, attn, name, args, cpu_seconds: float) -> dict:
    import numpy as np

    import oracle
    from io_aware_exact_amd.inputs import WORKLOADS, make_qkv, to_f64

    w = WORKLOADS[name]
    G = w.H // w.kv_heads
    log(f"[bench] {name} workload {w}: generating inputs")
    t0 = time.perf_counter()
    q, k, v = make_qkv(w)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    log(f"[bench] {name} inputs ready in {time.perf_counter() - t0:.1f}s")
    o = torch.empty_like(dq)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    splits = w.num_splits or attn.attn_decode_splits(w.B, w.H, w.kv_heads, w.Tkv, w.d)
    ws_bytes = attn.attn_decode_workspace_bytes(w.B, w.H, w.d, splits)
    ws = torch.empty(max(16, ws_bytes), dtype=torch.uint8, device="cuda")
    total, kv = decode_bytes(w)
    unsplit = None
    auto = None
    if w.num_splits > 0:
        # the same step with the library's automatic partition count, beside
        # the workload's fixed one
        pa = attn.attn_decode_splits(w.B, w.H, w.kv_heads, w.Tkv, w.d)
        if pa != w.num_splits:
            wsa = torch.empty(max(16, attn.attn_decode_workspace_bytes(w.B, w.H, w.d, pa)), dtype=torch.uint8,
                              device="cuda")
            ca = attn.prepared_decode(dq, dk, dv, o, lse, pa, wsa, w.scale)
            settle(torch, ca, args.settle_ms)
            msa, _ = time_leg(torch, ca, args.steps, args.warmup)
            auto = {"splits": pa, "ms_per_step": msa, "value": total / (msa * 1e-3) / 1e9,
                    "kernel": attn.attn_last_kernel()}
            del wsa
    if w.num_splits == 0:
        # the same step in one partition per (batch, head): the shape the
        # pages measured at batch 1
        c1 = attn.prepared_decode(dq, dk, dv, o, lse, 1, None, w.scale)
        settle(torch, c1, args.settle_ms)
        ms1, _ = time_leg(torch, c1, args.steps, args.warmup)
        unsplit = {"ms_per_step": ms1, "value": total / (ms1 * 1e-3) / 1e9, "kernel": attn.attn_last_kernel()}
    call = attn.prepared_decode(dq, dk, dv, o, lse, splits, ws, w.scale)
    settled = settle(torch, call, args.settle_ms)
    ms, nsteps = time_leg(torch, call, args.steps, args.warmup)
    kern = attn.attn_last_kernel()
    reps = time_repeats(torch, call, ms)
    gbps = total / (ms * 1e-3) / 1e9
    fn = attn.attn_decode_gqa if G > 1 else attn.attn_decode
    mem = measure_memory(torch, call, lambda: fn(dq, dk, dv, scale=w.scale, num_splits=splits),
                         dq.numel() * 2 + 2 * dk.numel() * 2, w.B * w.H * (w.d * 2 + 4), ws_bytes)
    # parity on sampled heads (oracle = the definition per head)
    rng = np.random.default_rng(5)
    errs_o, errs_l = [], []
    o_host, lse_host = o.cpu(), lse.cpu()
    for b, h in [(0, 0), (w.B - 1, w.H - 1)] + list(zip(rng.integers(0, w.B, 6).tolist(),
                                                        rng.integers(0, w.H, 6).tolist())):
        o_ref, lse_ref = oracle.attention(to_f64(q[b, h]), to_f64(k[b, h // G]), to_f64(v[b, h // G]), w.scale)
        errs_o.append(float(np.abs(to_f64(o_host[b, h]) - o_ref).max()))
        errs_l.append(float(abs(float(lse_host[b, h]) - lse_ref[0])))
    del dq, dk, dv, ws
    torch.cuda.empty_cache()
    cpu = None
    if cpu_seconds > 0:
        # oracle leg, bounded: query heads on the host until cpu_seconds
        done, t_cpu = 0, 0.0
        while t_cpu < cpu_seconds and done < w.B * w.H:
            b, h = done % w.B, (7 * done) % w.H
            qb, kb, vb = to_f64(q[b, h]), to_f64(k[b, h // G]), to_f64(v[b, h // G])
            t0 = time.perf_counter()
            oracle.attention(qb, kb, vb, w.scale)
            t_cpu += time.perf_counter() - t0
            done += 1
        cpu = {"value": done * (total / (w.B * w.H)) / t_cpu / 1e9, "unit": "GB/s", "cores": blas_threads(),
               "kind": "oracle", "seconds": t_cpu,
               "sample": f"{done} (batch, query head) slices, float64 numpy definition"}
    del q, k, v
    heads = f"H={w.H}" if G == 1 else f"Hq={w.H} Hkv={w.kv_heads}"
    plan = f"splits={splits}" if w.num_splits else f"splits=auto({splits})"
    out = {
        "workload": f"{name} B={w.B} {heads} Tq=1 Tkv={w.Tkv} d={w.d} bf16 {plan}",
        "metric": "decode attention KV-cache read bandwidth",
        "value": gbps,
        "unit": "GB/s",
        "kv_only_GBps": kv / (ms * 1e-3) / 1e9,
        "ms_per_step": ms,
        "steps": nsteps,
        "warmup": args.warmup,
        "settle_ms": settled,
        "kernel": kern,
        "algorithmic_bytes_per_call": total,
        "repeats": reps,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": gbps / PEAK_HBM_GBPS, "traffic": measured_traffic("decode", name, kern)},
        "parity": {"max_abs_err_o": max(errs_o), "max_abs_err_lse": max(errs_l), "tol_o": 2e-2, "tol_lse": 1e-3,
                   "ok": bool(max(errs_o) <= 2e-2 and max(errs_l) <= 1e-3), "heads_checked": len(errs_o)},
        "memory": mem,
        "extra_device_bytes": mem["extra_device_bytes"],
        "cpu_baseline": cpu,
    }
    if unsplit is not None:
        out["unsplit"] = unsplit
        out["speedup_vs_unsplit"] = unsplit["ms_per_step"] / ms
    if auto is not None:
        out["automatic_splits"] = auto
    return out


def run_backward(torch, attn, args, name="gpt2"):
    """The backward pass (attn_bwd) on a prefill workload: forward once for O
    and LSE, then time the three backward kernels; parity of dQ, dK, dV on
    sampled heads against the float64 backward oracle."""
    import numpy as np

    import oracle
    from io_aware_exact_amd.inputs import WORKLOADS, make_qkv, make_tensor, to_f64

    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    do = make_tensor(w.seed + 1000, "v", w.B, w.H, w.Tq, w.d, "bf16")
    dq_, dk_, dv_, ddo = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = attn.attn_fwd(dq_, dk_, dv_, causal=w.causal, scale=w.scale)
    gq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    gk = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    gv = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    ws_bytes = attn.attn_bwd_workspace_bytes(w.B, w.H, w.Tq)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    call = attn.prepared_bwd(dq_, dk_, dv_, o, lse, ddo, gq, gk, gv, w.causal, ws, w.scale)
    settled = settle(torch, call, args.settle_ms)
    ms, nsteps = time_leg(torch, call, args.steps, args.warmup)
    kern = attn.attn_last_kernel()
    reps = time_repeats(torch, call, ms)
    mem = measure_memory(torch, call, lambda: attn.attn_bwd(dq_, dk_, dv_, o, lse, ddo, causal=w.causal,
                                                            scale=w.scale),
                         5 * dq_.numel() * 2 + lse.numel() * 4, 3 * q.numel() * 4, ws_bytes)
    errs = []
    hq, hk, hv = gq.cpu(), gk.cpu(), gv.cpu()
    for b, h in [(0, 0), (w.B - 1, w.H - 1), (w.B // 2, w.H // 3)]:
        rq, rk, rv, _ = oracle.attention_backward(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]),
                                                  to_f64(do[b, h]), w.scale, w.causal)
        errs.append(max(float(np.abs(to_f64(g[b, h]) - r).max()) for g, r in ((hq, rq), (hk, rk), (hv, rv))))
    del dq_, dk_, dv_, ddo, o, lse, gq, gk, gv, ws
    torch.cuda.empty_cache()
    # model flops: the 5 products of the standard backward (S, dP, dV, dK, dQ), 2 d flops per pair each
    flops = 5 * 2 * w.B * w.H * w.d * visible_pairs(w.Tq, w.Tkv, w.causal)
    tf = flops / (ms * 1e-3) / 1e12
    return {
        "workload": f"{name} backward B={w.B} H={w.H} Tq={w.Tq} Tkv={w.Tkv} d={w.d} "
                    f"{'causal' if w.causal else 'non-causal'} bf16 in, fp32 dQ/dK/dV",
        "metric": "attn bwd TFLOP/s (5 products, causal-adjusted)",
        "value": tf,
        "unit": "TFLOP/s",
        "ms_per_step": ms,
        "steps": nsteps,
        "warmup": args.warmup,
        "settle_ms": settled,
        "kernel": kern,
        "repeats": reps,
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_BF16_TFLOPS, "traffic": measured_traffic("backward", name, kern)},
        "parity": {"max_abs_err_dq_dk_dv": max(errs), "heads_checked": len(errs)},
        "memory": mem,
        "extra_device_bytes": mem["extra_device_bytes"],
    }


def run_prefill_split(torch, attn, args, name="long_1head"):
    """Prefill on a shape with too few query tiles to fill the chip: attn_fwd
    (one workgroup per query tile) against attn_fwd_split (the key axis of
    long tiles split across workgroups, then merged), same inputs; parity of
    sampled rows against the float64 oracle."""
    import numpy as np

    import oracle
    from io_aware_exact_amd.inputs import WORKLOADS, make_qkv, to_f64

    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty_like(dq)
    lse = torch.empty((w.B, w.H, w.Tq), dtype=torch.float32, device="cuda")
    cp = attn.prepared_fwd(dq, dk, dv, o, lse, w.causal, w.scale)
    settle(torch, cp, args.settle_ms)
    ms_plain, _ = time_leg(torch, cp, args.steps, args.warmup)
    kern_plain = attn.attn_last_kernel()
    o_plain = o.clone()
    nbytes = attn.attn_fwd_split_workspace_bytes(w.B, w.H, w.Tq, w.Tkv, w.d, w.causal, 0)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    call = attn.prepared_fwd(dq, dk, dv, o, lse, w.causal, w.scale, kv_chunk=0, workspace=ws)
    settled = settle(torch, call, args.settle_ms)
    ms, nsteps = time_leg(torch, call, args.steps, args.warmup)
    kern = attn.attn_last_kernel()
    reps = time_repeats(torch, call, ms)
    diff = float((o.float() - o_plain.float()).abs().max())
    mem = measure_memory(torch, call, lambda: attn.attn_fwd_split(dq, dk, dv, causal=w.causal, scale=w.scale),
                         3 * dq.numel() * 2, prefill_output_bytes(w), nbytes)
    rows = sampled_rows(w.Tq, 512, np.random.default_rng(77))
    o_ref, lse_ref = oracle.attention(to_f64(q[0, 0]), to_f64(k[0, 0]), to_f64(v[0, 0]), w.scale, w.causal,
                                      rows=rows)
    oh, lh = o.cpu()[0, 0][rows], lse.cpu()[0, 0][rows]
    eo, el = float(np.abs(to_f64(oh) - o_ref).max()), float(np.abs(to_f64(lh) - lse_ref).max())
    flops = prefill_flops(w)
    del dq, dk, dv, ws, o_plain, o, lse
    torch.cuda.empty_cache()
    tf = flops / (ms * 1e-3) / 1e12
    return {
        "workload": workload_label(w) + ", key axis split across workgroups",
        "metric": "attn fwd TFLOP/s (causal-adjusted), key axis split across workgroups",
        "value": tf,
        "unit": "TFLOP/s",
        "ms_per_step": ms,
        "steps": nsteps,
        "warmup": args.warmup,
        "settle_ms": settled,
        "kernel": kern,
        "repeats": reps,
        "workspace_bytes": nbytes,
        "unsplit": {"ms_per_step": ms_plain, "value": flops / (ms_plain * 1e-3) / 1e12, "kernel": kern_plain},
        "speedup_vs_unsplit": ms_plain / ms,
        "max_abs_diff_vs_unsplit_o": diff,
        "parity": {"max_abs_err_o": eo, "max_abs_err_lse": el, "tol_o": 2e-2, "tol_lse": 1e-3,
                   "ok": bool(eo <= 2e-2 and el <= 1e-3), "rows_checked": int(rows.size)},
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_BF16_TFLOPS, "traffic": measured_traffic("prefill_split", name, kern)},
        "memory": mem,
        "extra_device_bytes": mem["extra_device_bytes"],
    }


# ------------------------------------------------------------------ ceilings

def achievable_ceilings(torch):
    """Measured ceilings beside the vendor peaks: a 1 GiB device copy (bytes
    read + written per second), a library bf16 GEMM (torch.mm, 8192^3) and the
    matrix-pipe probe."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms_copy = time_steps(torch, lambda: dst.copy_(src), 10, 2)
    del src, dst
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    ms_mm = time_steps(torch, lambda: torch.mm(a, b), 10, 2)
    del a, b
    torch.cuda.empty_cache()
    out = {"copy_GBps": 2 * (1 << 30) / (ms_copy * 1e-3) / 1e9,
           "copy": "torch device-to-device copy of 1 GiB, read + write bytes",
           "bf16_gemm_TFLOPs": 2 * n ** 3 / (ms_mm * 1e-3) / 1e12,
           "gemm": "torch.mm bf16 8192 x 8192 x 8192 (library GEMM)"}
    rate = mfma_loop_rate(torch)
    if rate is not None:
        out["mfma_loop_TFLOPs"] = rate
        out["mfma_loop"] = ("matrix-pipe probe (libattn_probe.so): 2048 workgroups of 4 waves, each wave 4 "
                            "independent chains of v_mfma_f32_32x32x16_bf16 from registers, 4096 steps")
    rates = instruction_rates(torch)
    if rates is not None:
        out["issue"] = rates
    return out


ISSUE_MODES = ("exp2_mul", "fma_mul", "mfma", "mfma_beside_exp2", "mfma_beside_fma", "prefill_block_mix",
               "lds_read_b128", "lds_read_b64_tr_b16", "exp2", "exp2_beside_fma", "fma32_mfma2", "fma32_mfma4",
               "fma32_mfma16x16x32_4", "fma32")
ISSUE_OPS = {"exp2_mul": 16, "fma_mul": 16, "mfma": 2}   # independent ops per loop iteration


def instruction_rates(torch, waves=(1, 2, 3), rounds: int = 8):
    """Issue and pipe rates from the instruction-mix probe of libattn_probe.so.
    For each mode and each count w of waves per SIMD (held there by an LDS
    reservation; `rounds` full rounds of CUs * w workgroups of 4 waves): the
    shader-clock cycles one SIMD spends per loop iteration of one wave (the
    event-timed launch over the wave-iterations each SIMD ran, times the clock
    the waves' s_memtime / s_memrealtime ratio shows), and that clock.  Derived
    at 3 waves per SIMD (the prefill kernels' occupancy): cycles per exp2+mul
    pair, per fma+mul pair, per 32x32x16 bf16 MFMA, the share of the
    prefill's per-block mix (16 MFMAs and the softmax of 32 scores per lane,
    from registers) that the matrix pipe is busy, the LDS read rate of a
    compute unit (conflict-free ds_read_b128, and ds_read_b64_tr_b16), and
    the issue-port time of an exp2, an FMA and each MFMA shape (what each
    adds to a loop of 32 independent FMAs).  None if the probe library is
    not built."""
    import ctypes

    path = os.path.join(ROOT, "io_aware_exact_amd", "libattn_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    if not hasattr(lib, "probe_issue"):
        return None
    lib.probe_issue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_issue.restype = ctypes.c_int
    threads = lib.probe_issue_threads()
    wpb = threads // 64
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ops = torch.full((lib.probe_issue_operand_bytes() // 2,), 0.0625, dtype=torch.bfloat16, device="cuda")
    blocks_max = cus * max(waves) * rounds
    out = torch.empty(blocks_max * threads, dtype=torch.float32, device="cuda")
    ticks = torch.empty(blocks_max * wpb * 2, dtype=torch.int64, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cycles, clock_mhz = {}, {}
    for mode, name in enumerate(ISSUE_MODES):
        iters = 256 if name == "prefill_block_mix" else 1024
        cycles[name], clock_mhz[name] = {}, {}
        for w in waves:
            blocks = cus * w * rounds

            def call():
                rc = lib.probe_issue(mode, w, blocks, iters, ctypes.c_void_p(ops.data_ptr()),
                                     ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ticks.data_ptr()), stream)
                if rc != 0:
                    raise RuntimeError(f"issue probe launch failed (hipError {rc})")

            ms = time_steps(torch, call, 3, 1)
            t = ticks[: blocks * wpb * 2].view(-1, 2).double().sum(0)
            mhz = 100.0 * t[0].item() / t[1].item()
            wave_iters_per_simd = blocks * wpb * iters / (4 * cus)
            cycles[name][str(w)] = ms * 1e-3 / wave_iters_per_simd * mhz * 1e6
            clock_mhz[name][str(w)] = mhz
    del ops, out, ticks
    w3 = str(max(waves))
    mfma = cycles["mfma"][w3] / ISSUE_OPS["mfma"]
    return {
        "simd_cycles_per_iteration": cycles,
        "clock_mhz": clock_mhz,
        "waves_per_simd": list(waves),
        "rounds": rounds,
        "cycles_per_exp2_mul": cycles["exp2_mul"][w3] / ISSUE_OPS["exp2_mul"],
        "cycles_per_fma_mul": cycles["fma_mul"][w3] / ISSUE_OPS["fma_mul"],
        "cycles_per_mfma_32x32x16_bf16": mfma,
        "prefill_block_mix_mfma_share": 16 * mfma / cycles["prefill_block_mix"][w3],
        # 4 SIMDs each finish one wave-iteration of 8 KiB of reads per that many cycles
        "lds_read_bytes_per_clk_per_cu": 4 * 8192 / cycles["lds_read_b128"][w3],
        "lds_read_tr_bytes_per_clk_per_cu": 4 * 8192 / cycles["lds_read_b64_tr_b16"][w3],
        # issue-port time: what an instruction adds to 32 independent FMAs
        "cycles_per_exp2": cycles["exp2"][w3] / 16,
        "exp2_beside_16_fma_over_sum": cycles["exp2_beside_fma"][w3] / (cycles["exp2"][w3] + cycles["fma32"][w3] / 2),
        "cycles_per_fma": cycles["fma32"][w3] / 32,
        "port_cycles_per_mfma_32x32x16_bf16": (cycles["fma32_mfma4"][w3] - cycles["fma32"][w3]) / 4,
        "port_cycles_per_mfma_16x16x32_bf16": (cycles["fma32_mfma16x16x32_4"][w3] - cycles["fma32"][w3]) / 4,
        "probe": ("instruction-mix probe (libattn_probe.so, issue_probe.hip): loops with no memory traffic, "
                  "w waves per SIMD held by an LDS reservation; modes " + ", ".join(ISSUE_MODES)),
    }


def mfma_loop_rate(torch, blocks: int = 2048, iters: int = 4096):
    """bf16 MFMA rate the chip sustains under load (TFLOP/s): the probe kernel
    of libattn_probe.so, timed with HIP events on the current stream; None if
    the probe library is not built."""
    import ctypes

    path = os.path.join(ROOT, "io_aware_exact_amd", "libattn_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.probe_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_mfma_loop.restype = ctypes.c_int
    lib.probe_mfma_loop_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.probe_mfma_loop_flops.restype = ctypes.c_double
    lib.probe_mfma_loop_threads.restype = ctypes.c_int
    out = torch.empty(blocks * lib.probe_mfma_loop_threads(), dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call():
        rc = lib.probe_mfma_loop(blocks, iters, ctypes.c_void_p(out.data_ptr()), stream)
        if rc != 0:
            raise RuntimeError(f"MFMA probe launch failed (hipError {rc})")

    ms = time_steps(torch, call, 10, 3)
    del out
    return lib.probe_mfma_loop_flops(blocks, iters) / (ms * 1e-3) / 1e12


# ------------------------------------------------------------------ main

def copy_calibration(torch) -> int:
    """Three device-to-device copies of 512 MiB: a kernel of known traffic
    that HBM byte counters are scaled by."""
    src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    n = src.numel()
    del src, dst
    torch.cuda.empty_cache()
    return n


def run_leg(torch, attn, leg, args, cpu_seconds: float) -> dict:
    if leg in PREFILL_LEGS:
        return run_prefill(torch, attn, leg, args, cpu_seconds, cold=(leg == "gpt2"))
    if leg in DECODE_LEGS:
        r = run_decode(torch, attn, leg, args, cpu_seconds)
        log(f"[bench] {leg} {r['kernel']}: {r['ms_per_step']:.3f} ms/step, {r['value']:.0f} GB/s")
        return r
    if leg == "backward":
        r = run_backward(torch, attn, args)
        log(f"[bench] backward {r['kernel']}: {r['ms_per_step'] * 1e3:.1f} us/step, {r['value']:.1f} TFLOP/s")
        return r
    r = run_prefill_split(torch, attn, args)
    log(f"[bench] prefill_split {r['kernel']}: {r['ms_per_step'] * 1e3:.1f} us/step "
        f"(unsplit {r['unsplit']['ms_per_step'] * 1e3:.1f} us)")
    return r


def parse_legs(spec: str, args) -> list:
    if spec in ("", "none"):
        legs = []
    elif spec == "all":
        legs = list(LEGS)
    else:
        legs = [s.strip() for s in spec.split(",") if s.strip()]
        bad = [s for s in legs if s not in LEGS]
        if bad:
            raise SystemExit(f"unknown legs {bad}; choose from {', '.join(LEGS)}")
    drop = set()
    if args.no_decode:
        drop |= set(DECODE_LEGS)
    if args.no_split:
        drop.add("prefill_split")
    if args.no_extra:
        drop.add("mid_d128")
    if args.no_backward:
        drop.add("backward")
    return [x for x in legs if x not in drop]


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="back-to-back calls before each leg's warm-up so its timed steps start at a settled clock")
    ap.add_argument("--workload", default=HEADLINE, help="headline prefill workload (long, mid, mid_causal, gpt2, tiny)")
    ap.add_argument("--legs", default="all", help=f"comma list of legs to run beside the headline ({', '.join(LEGS)}), "
                                                  "'all' or 'none'")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode legs")
    ap.add_argument("--no-split", action="store_true", help="skip the split-prefill leg")
    ap.add_argument("--no-extra", action="store_true", help="skip the head-width-128 prefill leg")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward leg")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing legs")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the copy / GEMM / matrix-pipe ceilings")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle leg of the headline: seconds of CPU work")
    ap.add_argument("--leg-cpu-seconds", type=float, default=3.0, help="oracle leg of each other leg: seconds")
    ap.add_argument("--legs-only", action="store_true",
                    help="run only the legs (no headline line): for profiling one leg's kernels on their own")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 3 device-to-device copies of 512 MiB (a reference for HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library has no multi-GPU path (each GPU would run its own shard; see the sharding design).",
              file=sys.stderr)
        sys.exit(2)
    legs = parse_legs(args.legs, args)

    import torch

    import io_aware_exact_amd as attn

    if not os.path.exists(attn.attn.LIB_PATH):
        from io_aware_exact_amd import build as _build
        _build.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    cpu_main = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    cpu_leg = 0.0 if args.no_cpu_baseline else args.leg_cpu_seconds

    if args.legs_only:
        out = {"legs": {leg: run_leg(torch, attn, leg, args, cpu_leg) for leg in legs}}
        if args.copy_calibration:
            out["copy_calibration_bytes"] = copy_calibration(torch)
        out["kernel_sources_digest"] = kernel_sources_digest()
        print(json.dumps(out), flush=True)
        return
    head = run_prefill(torch, attn, args.workload, args, cpu_main, cold=True, headline=True)
    props = torch.cuda.get_device_properties(0)
    result = {
        "metric": "attn fwd TFLOP/s (causal-adjusted) & % bf16 MFMA peak (prefill); decode KV GB/s & % HBM peak",
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if head["workload"].endswith("bf16") else "f32",
        "data": "synthetic",
        "config": {"workload": head["workload"], "parallelism": "none (1 GPU)"},
        "kernel": head["kernel"],
        "pct_of_peak": head["pct_of_peak"],
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "parity": head["parity"],
        "repeats": head["repeats"],
        "settle_ms": head["settle_ms"],
        "cold_cache": head.get("cold_cache"),
        "memory": head["memory"],
        "extra_device_bytes": head["extra_device_bytes"],
        "device": {"name": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", ""),
                   "compute_units": props.multi_processor_count, "hip": torch.version.hip,
                   "max_clock_mhz": device_max_clock_mhz()},
        "context": {"pages": "17.3 TFLOP/s (fp16, B=1 H=12 d=64 causal, T=8192) and 24 MiB peak extra memory "
                             "at T=16384 for the memory-efficient kernel on a 12 GiB compute-capability-7.5 GPU; "
                             "another machine's numbers, not the target"},
    }
    from io_aware_exact_amd.inputs import WORKLOADS
    w = WORKLOADS[args.workload]
    result["config"].update({"B": w.B, "H": w.H, "Tq": w.Tq, "Tkv": w.Tkv, "d": w.d, "causal": w.causal,
                             "scale": w.scale})
    result["legs"] = {}
    for leg in legs:
        result["legs"][leg] = run_leg(torch, attn, leg, args, cpu_leg)
    legs_run = result["legs"]
    if "mid" in legs_run and "mid_causal" in legs_run:
        t_full = legs_run["mid"]["repeats"]["median_ms"]
        t_causal = legs_run["mid_causal"]["repeats"]["median_ms"]
        result["causal_to_full_time"] = {"mid": t_causal / t_full, "work_ratio": 4096 * 4097 / 2 / 4096 ** 2,
                                         "pages": PAGES_CAUSAL_RATIO,
                                         "note": "mid_causal over mid, medians of the 50 ms repeats"}
    if not args.no_ceilings:
        ceil = achievable_ceilings(torch)
        if "mfma_loop_TFLOPs" in ceil:
            ceil["headline_frac_of_mfma_loop"] = head["value"] / ceil["mfma_loop_TFLOPs"]
        ceil["headline_frac_of_gemm"] = head["value"] / ceil["bf16_gemm_TFLOPs"]
        if "decode" in legs_run:
            ceil["decode_frac_of_copy"] = legs_run["decode"]["value"] / ceil["copy_GBps"]
        result["achievable"] = ceil
        log(f"[bench] achievable: copy {ceil['copy_GBps']:.0f} GB/s, bf16 GEMM {ceil['bf16_gemm_TFLOPs']:.0f} TFLOP/s,"
            f" MFMA loop {ceil.get('mfma_loop_TFLOPs', float('nan')):.0f} TFLOP/s")
        if "issue" in ceil:
            iss = ceil["issue"]
            log(f"[bench] issue probe (3 waves/SIMD): exp2+mul {iss['cycles_per_exp2_mul']:.2f}, fma+mul "
                f"{iss['cycles_per_fma_mul']:.2f}, MFMA {iss['cycles_per_mfma_32x32x16_bf16']:.1f} cycles; "
                f"prefill block mix keeps the matrix pipe {100 * iss['prefill_block_mix_mfma_share']:.0f}% busy; "
                f"LDS reads {iss['lds_read_bytes_per_clk_per_cu']:.0f} B/clk per CU "
                f"({iss['lds_read_tr_bytes_per_clk_per_cu']:.0f} transposing)")
    if args.copy_calibration:
        result["copy_calibration_bytes"] = copy_calibration(torch)
    result["kernel_sources_digest"] = kernel_sources_digest()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
