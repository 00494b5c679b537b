"""Calls from several streams and several host threads at once.

The library keeps no state between calls except two thread-local strings (the
last kernel's name and the last error's detail), takes every buffer from the
caller and enqueues on the caller's stream.  So calls on different streams
may overlap on the GPU, and host threads may call it concurrently (the ctypes
binding releases the interpreter lock during each call), each seeing its own
kernel names.  Each test compares against the same calls made one at a time
on one stream; the kernels are deterministic, so the comparison is bitwise.
"""

import sys
import threading

import pytest
import torch

import io_aware_exact_amd as attn

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16).cuda()


def job(kind, seed):
    """A callable that runs one entry point on inputs made here (on the current
    stream) and returns its outputs."""
    if kind == "prefill64":
        q, k, v = (rand((2, 4, 700, 64), seed + i) for i in range(3))
        return lambda: attn.attn_fwd(q, k, v, causal=True)
    if kind == "prefill128":
        q, k, v = (rand((1, 4, 500, 128), seed + i) for i in range(3))
        return lambda: attn.attn_fwd(q, k, v, causal=False)
    if kind == "decode":
        q = rand((4, 16, 1, 128), seed)
        k, v = rand((4, 4, 3000, 128), seed + 1), rand((4, 4, 3000, 128), seed + 2)
        return lambda: attn.attn_decode_gqa(q, k, v, num_splits=0)
    if kind == "backward":
        q, k, v, do = (rand((1, 3, 300, 64), seed + i) for i in range(4))

        def run():
            o, lse = attn.attn_fwd(q, k, v, causal=True)
            return attn.attn_bwd(q, k, v, o, lse, do, causal=True)
        return run
    raise ValueError(kind)


KINDS = ["prefill64", "prefill128", "decode", "backward"]


def reference(kinds):
    """Outputs and kernel names of each job run alone on the default stream."""
    out = {}
    for i, kind in enumerate(kinds):
        run = job(kind, 10 * i)
        res = run()
        torch.cuda.synchronize()
        out[kind] = ([t.clone() for t in res], attn.attn_last_kernel())
    return out


def test_two_streams_overlap():
    ref = reference(["prefill64", "decode"])
    say("case two streams: prefill64 and decode")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        run1 = job("prefill64", 0)
    with torch.cuda.stream(s2):
        run2 = job("decode", 10)
    torch.cuda.synchronize()
    for rep in range(3):
        with torch.cuda.stream(s1):
            r1 = run1()
        with torch.cuda.stream(s2):
            r2 = run2()
        torch.cuda.synchronize()          # both enqueued before either is waited for
        for got, want in ((r1, ref["prefill64"][0]), (r2, ref["decode"][0])):
            assert all(torch.equal(a, b) for a, b in zip(got, want)), f"replay {rep}"


def test_host_threads_concurrently():
    ref = reference(KINDS)
    say("case four host threads: " + ", ".join(KINDS))
    results, names, errors = {}, {}, []
    start = threading.Barrier(len(KINDS))

    def worker(i, kind):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                run = job(kind, 10 * i)
                stream.synchronize()
                start.wait(timeout=60)
                seen = set()
                for _ in range(20):
                    res = run()
                    seen.add(attn.attn_last_kernel())
                stream.synchronize()
            results[kind] = [t.clone() for t in res]
            names[kind] = seen
        except Exception as e:          # reported below, in the main thread
            errors.append(f"{kind}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i, kind), daemon=True) for i, kind in enumerate(KINDS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
    for kind in KINDS:
        want, want_name = ref[kind]
        assert all(torch.equal(a, b) for a, b in zip(results[kind], want)), kind
        # each thread only ever saw the names of its own calls
        assert names[kind] == {want_name}, (kind, names[kind], want_name)
        say(f"  {kind}: {want_name}")
