#!/usr/bin/env python3
"""Benchmark of the exact attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gpt2]

Prints ONE JSON line on stdout (progress goes to stderr).  A step is one call
of the attention forward over one batch of the workload (default: GPT-2-shaped
causal prefill, B=4, H=12, T=1024, d=64, bf16): the prefill kernel runs every
prefill step of the hot path (Q tile load, K/V streaming, both products, the
online softmax, causal skipping, the epilogue).  The decode half of the path
(split-KV kernel + combine) is timed the same way on its own workload
(B=64, H=32, T_kv=8192, d=128, 16 partitions) and reported in "decode", and
its grouped-query form (the same step with 8 key/value heads for the 32 query
heads) in "decode_gqa"; both also report the same step with the library's
automatically chosen partition count ("automatic_splits").  "decode_b1" is
one sequence (12 heads of 64, 16K keys) with automatically chosen partitions
against one partition per head.
"mid_d128" is the mid-length prefill at head width 128; "backward" is the
backward pass (attn_bwd) on the GPT-2-shaped workload.
"prefill_split" times one 16K-token causal head, a
shape with too few query tiles to fill the chip, with and without the key
axis split across workgroups.

Inputs are seeded synthetic tensors already resident in HBM when timing
starts; W untimed warm-up steps (default 1000, ≈ 15 ms of GPT-2-shaped
calls: the first ≈ 8 ms of back-to-back calls after an idle host phase run
slower while the clock settles) are followed by exactly K timed steps
(default 2000, ≈ 30 ms),
bracketed by device synchronisation, with HIP events recorded on the stream
the kernels are launched on.  "repeats" times the headline prefill and each
decode step again as three repeats of at least 50 ms of back-to-back calls
(per-call median and spread).  The float64 oracle is timed on the host cores on
a bounded sample (the "cpu_baseline" leg) and checks the GPU output.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PEAK_F32_VALU_TFLOPS = 157.3  # MI355X fp32 vector (256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2 (packed) x 2.4 GHz)
PROFILES = os.path.join(ROOT, "profiles")


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


def decode_bytes(w) -> tuple[int, int]:
    """(all bytes, K/V-cache bytes) one decode step must move: K and V once
    (kv_heads of them), q in, O and LSE out."""
    kv = 2 * w.B * w.kv_heads * w.Tkv * w.d * 2
    return kv + 2 * w.B * w.H * w.d * 2 + w.B * w.H * 4, kv


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


def achievable_ceilings(torch):
    """Measured ceilings beside the vendor peaks: a 1 GiB device copy (bytes
    read + written per second) and a library bf16 GEMM (torch.mm, 8192^3)."""
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
    return out


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


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def cpu_baseline_prefill(w, q, k, v, o_gpu, lse_gpu, min_seconds: float):
    """Oracle leg: the float64 oracle on the host, over whole (b, h) heads of
    the same inputs until about ``min_seconds`` of CPU work is done; also the
    parity of the GPU output on those heads."""
    import numpy as np

    import oracle
    from io_aware_exact_amd.inputs import to_f64

    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, t_compute, t_convert, err_o, err_l = 0, 0.0, 0.0, 0.0, 0.0
    t_wall0 = time.perf_counter()
    while t_compute < min_seconds:
        b, h = heads[done % len(heads)]
        t0 = time.perf_counter()
        qb, kb, vb = to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h])
        t_convert += time.perf_counter() - t0
        t0 = time.perf_counter()
        o_ref, lse_ref = oracle.attention(qb, kb, vb, w.scale, w.causal)
        t_compute += time.perf_counter() - t0
        if done < len(heads):
            err_o = max(err_o, float(np.abs(to_f64(o_gpu[b, h]) - o_ref).max()))
            err_l = max(err_l, float(np.abs(to_f64(lse_gpu[b, h]) - lse_ref).max()))
        done += 1
    passes = done / len(heads)
    per_head = 4 * w.d * visible_pairs(w.Tq, w.Tkv, w.causal)
    value = per_head * done / t_compute / 1e12
    return {
        "value": value,
        "unit": "TFLOP/s",
        "cores": blas_threads(),
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{done} (batch, head) slices of this workload ({passes:.2f} x its {len(heads)} slices), "
                  f"float64 numpy, full T_q x T_kv scores materialised per head; causal-adjusted flop count",
        "seconds": t_compute,
        "conversion_seconds": t_convert,
        "wall_seconds": time.perf_counter() - t_wall0,
    }, {"max_abs_err_o": err_o, "max_abs_err_lse": err_l, "heads_checked": min(done, len(heads))}


def run_decode(torch, attn, steps, warmup, name="decode"):
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
    ws = torch.empty(max(16, attn.attn_decode_workspace_bytes(w.B, w.H, w.d, splits)), dtype=torch.uint8,
                     device="cuda")
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
            msa = time_steps(torch, attn.prepared_decode(dq, dk, dv, o, lse, pa, wsa, w.scale), steps, warmup)
            auto = {"splits": pa, "ms_per_step": msa, "value": total / (msa * 1e-3) / 1e9,
                    "kernel": attn.attn_last_kernel()}
            del wsa
    if w.num_splits == 0:
        # the same step in one partition per (batch, head): the shape the
        # pages measured at batch 1
        ms1 = time_steps(torch, attn.prepared_decode(dq, dk, dv, o, lse, 1, None, w.scale), steps, warmup)
        unsplit = {"ms_per_step": ms1, "value": total / (ms1 * 1e-3) / 1e9, "kernel": attn.attn_last_kernel()}
    call = attn.prepared_decode(dq, dk, dv, o, lse, splits, ws, w.scale)
    ms = time_steps(torch, call, steps, warmup)
    kern = attn.attn_last_kernel()
    reps = time_repeats(torch, call, ms)
    gbps = total / (ms * 1e-3) / 1e9
    # parity on sampled heads (oracle = the definition per head)
    rng = np.random.default_rng(5)
    errs_o, errs_l = [], []
    for b, h in [(0, 0), (w.B - 1, w.H - 1)] + list(zip(rng.integers(0, w.B, 6).tolist(), rng.integers(0, w.H, 6).tolist())):
        o_ref, lse_ref = oracle.attention(to_f64(q[b, h]), to_f64(k[b, h // G]), to_f64(v[b, h // G]), w.scale)
        errs_o.append(float(np.abs(to_f64(o[b, h]) - o_ref).max()))
        errs_l.append(float(abs(float(lse[b, h]) - lse_ref[0])))
    # oracle leg, bounded: a few query heads on the host
    sample_heads = 32
    t0 = time.perf_counter()
    for i in range(sample_heads):
        b, h = i % w.B, (7 * i) % w.H
        oracle.attention(to_f64(q[b, h]), to_f64(k[b, h // G]), to_f64(v[b, h // G]), w.scale)
    t_cpu = time.perf_counter() - t0
    cpu_gbps = sample_heads * (total / (w.B * w.H)) / t_cpu / 1e9
    del dq, dk, dv, q, k, v
    torch.cuda.empty_cache()
    heads = f"H={w.H}" if G == 1 else f"Hq={w.H} Hkv={w.kv_heads}"
    plan = f"splits={splits}" if w.num_splits else f"splits=auto({splits})"
    out = {
        "workload": f"{name} B={w.B} {heads} Tq=1 Tkv={w.Tkv} d={w.d} bf16 {plan}",
        "metric": "decode attention KV-cache read bandwidth",
        "value": gbps,
        "unit": "GB/s",
        "kv_only_GBps": kv / (ms * 1e-3) / 1e9,
        "ms_per_step": ms,
        "steps": steps,
        "warmup": warmup,
        "kernel": kern,
        "repeats": reps,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": gbps / PEAK_HBM_GBPS, "traffic": measured_traffic("decode", name, kern)},
        "parity": {"max_abs_err_o": max(errs_o), "max_abs_err_lse": max(errs_l), "heads_checked": len(errs_o)},
        "cpu_baseline": {"value": cpu_gbps, "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
                         "sample": f"{sample_heads} (batch, query head) slices, float64 numpy definition"},
    }
    if unsplit is not None:
        out["unsplit"] = unsplit
        out["speedup_vs_unsplit"] = unsplit["ms_per_step"] / ms
    if auto is not None:
        out["automatic_splits"] = auto
    return out


def run_prefill(torch, attn, steps, warmup, name):
    """Another prefill workload, timed like the main one (no oracle leg)."""
    from io_aware_exact_amd.inputs import WORKLOADS, make_qkv

    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty_like(dq)
    lse = torch.empty((w.B, w.H, w.Tq), dtype=torch.float32, device="cuda")
    ms = time_steps(torch, attn.prepared_fwd(dq, dk, dv, o, lse, w.causal, w.scale), steps, warmup)
    kern = attn.attn_last_kernel()
    del dq, dk, dv, o, lse
    torch.cuda.empty_cache()
    tf = prefill_flops(w) / (ms * 1e-3) / 1e12
    return {
        "workload": f"{name} prefill B={w.B} H={w.H} Tq={w.Tq} Tkv={w.Tkv} d={w.d} "
                    f"{'causal' if w.causal else 'non-causal'} bf16",
        "metric": "attn fwd TFLOP/s (causal-adjusted)",
        "value": tf,
        "unit": "TFLOP/s",
        "ms_per_step": ms,
        "kernel": kern,
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_BF16_TFLOPS, "traffic": measured_traffic("prefill", name, kern)},
    }


def run_backward(torch, attn, steps, warmup, name="gpt2"):
    """The backward pass (attn_bwd) on a prefill workload: forward once for O
    and LSE, then time the three backward kernels; parity of dV on sampled
    heads against the float64 backward oracle."""
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
    ws = torch.empty(attn.attn_bwd_workspace_bytes(w.B, w.H, w.Tq), dtype=torch.uint8, device="cuda")
    call = attn.prepared_bwd(dq_, dk_, dv_, o, lse, ddo, gq, gk, gv, w.causal, ws, w.scale)
    ms = time_steps(torch, call, steps, warmup)
    kern = attn.attn_last_kernel()
    errs = []
    for b, h in [(0, 0), (w.B - 1, w.H - 1), (w.B // 2, w.H // 3)]:
        rq, rk, rv, _ = oracle.attention_backward(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]),
                                                  to_f64(do[b, h]), w.scale, w.causal)
        errs.append(max(float(np.abs(to_f64(g[b, h]) - r).max()) for g, r in ((gq, rq), (gk, rk), (gv, rv))))
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
        "kernel": kern,
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_BF16_TFLOPS, "traffic": measured_traffic("backward", name, kern)},
        "parity": {"max_abs_err_dq_dk_dv": max(errs), "heads_checked": len(errs)},
    }


def run_prefill_split(torch, attn, steps, warmup, name="long_1head"):
    """Prefill on a shape with too few query tiles to fill the chip: attn_fwd
    (one workgroup per query tile) against attn_fwd_split (the key axis of
    long tiles split across workgroups, then merged), same inputs."""
    from io_aware_exact_amd.inputs import WORKLOADS, make_qkv

    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty_like(dq)
    lse = torch.empty((w.B, w.H, w.Tq), dtype=torch.float32, device="cuda")
    ms_plain = time_steps(torch, attn.prepared_fwd(dq, dk, dv, o, lse, w.causal, w.scale), steps, warmup)
    kern_plain = attn.attn_last_kernel()
    o_plain = o.clone()
    nbytes = attn.attn_fwd_split_workspace_bytes(w.B, w.H, w.Tq, w.Tkv, w.d, w.causal, 0)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    call = attn.prepared_fwd(dq, dk, dv, o, lse, w.causal, w.scale, kv_chunk=0, workspace=ws)
    ms = time_steps(torch, call, steps, warmup)
    kern = attn.attn_last_kernel()
    diff = float((o.float() - o_plain.float()).abs().max())
    flops = prefill_flops(w)
    del dq, dk, dv, ws, o_plain
    torch.cuda.empty_cache()
    tf = flops / (ms * 1e-3) / 1e12
    return {
        "workload": f"{name} prefill B={w.B} H={w.H} Tq={w.Tq} Tkv={w.Tkv} d={w.d} "
                    f"{'causal' if w.causal else 'non-causal'} bf16",
        "metric": "attn fwd TFLOP/s (causal-adjusted), key axis split across workgroups",
        "value": tf,
        "unit": "TFLOP/s",
        "ms_per_step": ms,
        "kernel": kern,
        "workspace_bytes": nbytes,
        "unsplit": {"ms_per_step": ms_plain, "value": flops / (ms_plain * 1e-3) / 1e12, "kernel": kern_plain},
        "speedup_vs_unsplit": ms_plain / ms,
        "max_abs_diff_vs_unsplit_o": diff,
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_BF16_TFLOPS, "traffic": measured_traffic("prefill_split", name, kern)},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="gpt2", help="prefill workload: gpt2, mid, mid_causal, long, tiny")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurements")
    ap.add_argument("--no-split", action="store_true", help="skip the split-prefill measurement")
    ap.add_argument("--no-extra", action="store_true", help="skip the head-width-128 prefill measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache prefill calls")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle leg: seconds of CPU work")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 3 device-to-device copies of 512 MiB (a reference for HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library has no multi-GPU path (each GPU would run its own shard; see the sharding design).", file=sys.stderr)
        sys.exit(2)

    import torch

    import io_aware_exact_amd as attn
    from io_aware_exact_amd.inputs import WORKLOADS, make_qkv

    if not os.path.exists(attn.attn.LIB_PATH):
        from io_aware_exact_amd import build as _build
        _build.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    w = WORKLOADS[args.workload]
    log(f"[bench] prefill workload {w}")
    q, k, v = make_qkv(w)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty_like(dq)
    lse = torch.empty((w.B, w.H, w.Tq), dtype=torch.float32, device="cuda")
    call = attn.prepared_fwd(dq, dk, dv, o, lse, w.causal, w.scale, f32=(w.dtype == "f32"))
    ms = time_steps(torch, call, args.steps, args.warmup)
    kern = attn.attn_last_kernel()
    reps = time_repeats(torch, call, ms)
    flops = prefill_flops(w)
    nbytes = prefill_bytes(w)
    tflops = flops / (ms * 1e-3) / 1e12
    # bf16 products run on the matrix cores; the fp32 path's are VALU FMAs
    compute_peak, compute_bound = ((PEAK_BF16_TFLOPS, "mfma") if w.dtype == "bf16"
                                   else (PEAK_F32_VALU_TFLOPS, "alu"))
    t_mfma = flops / (compute_peak * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBPS * 1e9)
    if t_hbm > t_mfma:
        ach = nbytes / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBPS}
    else:
        roof = {"bound": compute_bound, "achieved": tflops, "peak": compute_peak, "unit": "TFLOP/s",
                "frac": tflops / compute_peak}
    roof["traffic"] = measured_traffic("prefill", w.name, kern)
    log(f"[bench] prefill {kern}: {ms * 1e3:.2f} us/step, {tflops:.1f} TFLOP/s")
    cold = None
    if not args.no_cold:
        cold_ms, cold_min, cold_max = time_cold(torch, call)
        log(f"[bench] prefill with caches scrubbed between calls: {cold_ms * 1e3:.2f} us/call")
        cold = {"ms_per_call": cold_ms, "min_ms": cold_min, "max_ms": cold_max,
                "value": flops / (cold_ms * 1e-3) / 1e12, "unit": "TFLOP/s",
                "protocol": "512 MiB write before each call, per-call HIP events, median of 30"}
    props = torch.cuda.get_device_properties(0)

    result = {
        "metric": "attn fwd TFLOP/s (causal-adjusted) & % bf16 MFMA peak (prefill); decode KV GB/s & % HBM peak",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name} prefill B={w.B} H={w.H} Tq={w.Tq} Tkv={w.Tkv} d={w.d} "
                               f"{'causal' if w.causal else 'non-causal'} {w.dtype}",
                   "B": w.B, "H": w.H, "Tq": w.Tq, "Tkv": w.Tkv, "d": w.d, "causal": w.causal,
                   "scale": w.scale, "parallelism": "none (1 GPU)"},
        "kernel": kern,
        "pct_of_peak": {("bf16_mfma" if w.dtype == "bf16" else "f32_valu"): 100.0 * tflops / compute_peak,
                        "hbm_algorithmic": 100.0 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS},
        "roofline": roof,
        "repeats": reps,
        "cold_cache": cold,
        "extra_device_bytes": 0,
        "device": {"name": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", ""),
                   "compute_units": props.multi_processor_count, "hip": torch.version.hip},
    }
    if not args.no_cpu_baseline:
        log("[bench] oracle leg on the host")
        torch.cuda.synchronize()
        cpu, parity = cpu_baseline_prefill(w, q, k, v, o.cpu(), lse.cpu(), args.cpu_seconds)
        result["cpu_baseline"] = cpu
        result["parity"] = parity
        log(f"[bench] oracle {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads; parity {parity}")
    else:
        result["cpu_baseline"] = None
    del dq, dk, dv
    torch.cuda.empty_cache()
    if not args.no_extra:
        for name in ("mid_d128",):
            result[name] = run_prefill(torch, attn, args.steps, args.warmup, name)
            log(f"[bench] {name} {result[name]['kernel']}: {result[name]['ms_per_step'] * 1e3:.1f} us/step, "
                f"{result[name]['value']:.1f} TFLOP/s")
    if not args.no_backward:
        result["backward"] = run_backward(torch, attn, args.steps, args.warmup)
        log(f"[bench] backward {result['backward']['kernel']}: {result['backward']['ms_per_step'] * 1e3:.1f} us/step, "
            f"{result['backward']['value']:.1f} TFLOP/s")
    if not args.no_split:
        result["prefill_split"] = run_prefill_split(torch, attn, args.steps, args.warmup)
        log(f"[bench] prefill_split {result['prefill_split']['kernel']}: "
            f"{result['prefill_split']['ms_per_step'] * 1e3:.1f} us/step "
            f"(unsplit {result['prefill_split']['unsplit']['ms_per_step'] * 1e3:.1f} us)")
    if not args.no_decode:
        for name in ("decode", "decode_gqa", "decode_b1"):
            result[name] = run_decode(torch, attn, args.steps, args.warmup, name)
            log(f"[bench] {name} {result[name]['kernel']}: {result[name]['ms_per_step']:.3f} ms/step, "
                f"{result[name]['value']:.0f} GB/s")
    ceil = achievable_ceilings(torch)
    ceil["prefill_frac_of_gemm"] = tflops / ceil["bf16_gemm_TFLOPs"]
    if "mfma_loop_TFLOPs" in ceil:
        ceil["prefill_frac_of_mfma_loop"] = tflops / ceil["mfma_loop_TFLOPs"]
        if "mid_d128" in result:
            ceil["mid_d128_frac_of_mfma_loop"] = result["mid_d128"]["value"] / ceil["mfma_loop_TFLOPs"]
    if "decode" in result:
        ceil["decode_frac_of_copy"] = result["decode"]["value"] / ceil["copy_GBps"]
    result["achievable"] = ceil
    log(f"[bench] achievable: copy {ceil['copy_GBps']:.0f} GB/s, bf16 GEMM {ceil['bf16_gemm_TFLOPs']:.0f} TFLOP/s, "
        f"MFMA loop {ceil.get('mfma_loop_TFLOPs', float('nan')):.0f} TFLOP/s")
    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = src.numel()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
