"""The allocation-free decode entry point (attn_decode_noalloc) through the C ABI.

It must give what attn_decode_gqa gives with a caller workspace (the same
kernels, so bitwise equal), match the float64 oracle within the decode bars,
and take no device memory: neither the caching allocator nor the device's
free memory moves across a call.  Two calls in a row share the library's
per-device scratch, the second on a smaller input; the first fills nearly
all of the scratch.
"""

import sys

import numpy as np
import pytest
import torch

import io_aware_exact_amd as attn
import oracle
from io_aware_exact_amd.inputs import make_tensor, to_f64

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def inputs(seed, B, Hq, Hkv, Tkv, d):
    q = make_tensor(seed, "q", B, Hq, 1, d, "bf16")
    k = make_tensor(seed, "k", B, Hkv, Tkv, d, "bf16")
    v = make_tensor(seed, "v", B, Hkv, Tkv, d, "bf16")
    return q, k, v


def check_call(seed, B, Hq, Hkv, Tkv, d, splits, heads):
    say(f"case noalloc seed={seed} B={B} Hq={Hq} Hkv={Hkv} Tkv={Tkv} d={d} splits={splits}")
    scale = 1.0 / np.sqrt(d)
    q, k, v = inputs(seed, B, Hq, Hkv, Tkv, d)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o_ws, lse_ws = attn.attn_decode_gqa(dq, dk, dv, scale=scale, num_splits=splits)
    kern_ws = attn.attn_last_kernel()
    o = torch.empty_like(dq)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    alloc0 = torch.cuda.memory_allocated()
    free0 = torch.cuda.mem_get_info()[0]
    attn.attn_decode_noalloc(dq, dk, dv, o, lse, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    kern = attn.attn_last_kernel()
    assert torch.cuda.memory_allocated() == alloc0
    assert torch.cuda.mem_get_info()[0] == free0
    say(f"  kernel {kern}")
    assert kern == kern_ws
    assert torch.equal(o, o_ws), "output differs from the workspace entry point"
    assert torch.equal(lse, lse_ws), "lse differs from the workspace entry point"
    G = Hq // Hkv
    oh, lh = o.cpu(), lse.cpu()
    for b, h in heads:
        o_ref, lse_ref = oracle.attention(to_f64(q[b, h]), to_f64(k[b, h // G]), to_f64(v[b, h // G]), scale)
        eo = float(np.abs(to_f64(oh[b, h]) - o_ref).max())
        el = float(abs(float(lh[b, h]) - lse_ref[0]))
        assert eo <= 2e-2 and el <= 1e-3, (b, h, eo, el)
    say(f"  equal to attn_decode_gqa; oracle parity on {len(heads)} heads")


def test_noalloc_matches_workspace_entry_twice():
    cap = attn.attn_decode_noalloc_max_bytes()
    assert cap == 32 << 20
    # first call: 31.9 MB of partials, nearly the whole scratch (VALU kernel)
    need = attn.attn_decode_workspace_bytes(64, 32, 128, 30)
    assert cap - (2 << 20) < need <= cap
    check_call(31, 64, 32, 32, 600, 128, 30, [(0, 0), (63, 31), (17, 5), (40, 22)])
    # second call, smaller, grouped query heads on the matrix-core kernel: it
    # reads only records it wrote itself, whatever the first call left
    check_call(32, 2, 8, 2, 1000, 64, 7, [(0, 0), (1, 7), (1, 3)])
    # one partition: no scratch involved
    check_call(33, 3, 4, 4, 513, 64, 1, [(0, 0), (2, 3)])


def test_noalloc_refuses_partials_larger_than_the_scratch():
    q, k, v = inputs(34, 64, 32, 32, 64, 128)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty_like(dq)
    # 64 x 32 x 64 partitions x 130 floats = 68 MB > 32 MiB; clamped to Tkv = 64
    with pytest.raises(ValueError, match="scratch"):
        attn.attn_decode_noalloc(dq, dk, dv, o, None, num_splits=64)
