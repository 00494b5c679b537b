"""Parity of the HIP backward (attn_bwd, through the C ABI) with the float64
backward oracle.

Inputs: the seeded bf16 q, k, v of io_aware_exact_amd.inputs and an upstream
gradient dO drawn the same way (tensor stream "v" of seed + 1000, so it is
independent of q, k, v).  The forward runs on the GPU (attn_fwd) and its bf16
O and fp32 LSE feed the backward, as in training.  The oracle sees exactly the
bf16-rounded q, k, v, dO and computes the gradients of the definition in
float64 (it does not use the GPU's O or LSE).

Tolerance: max-abs error <= 2e-2 * max(1, max|reference|) per gradient.
Derivation: P and dS enter the MFMA products rounded to bf16 (relative error
at most 2^-8 per term, the unit roundoff of an 8-bit significand); the
forward's O, used for the row constant D, carries
the same rounding; summed over up to T_q rows with independent signs the
relative error of a gradient entry stays a small multiple of 2^-8 = 3.9e-3, and
the bound keeps a 5x margin over that, the same margin as the forward's 2e-2
bf16 bar on O.
"""

import sys

import numpy as np
import pytest
import torch

import io_aware_exact_amd as attn
import oracle
from io_aware_exact_amd.inputs import WORKLOADS, Workload, make_qkv, make_tensor, to_f64

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def upstream(w: Workload):
    return make_tensor(w.seed + 1000, "v", w.B, w.H, w.Tq, w.d, "bf16")


def tol(ref):
    return 2e-2 * max(1.0, float(np.abs(ref).max()))


def check(w: Workload):
    say(f"case {w}")
    q, k, v = make_qkv(w)
    do = upstream(w)
    dq_, dk_, dv_, ddo = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = attn.attn_fwd(dq_, dk_, dv_, causal=w.causal, scale=w.scale)
    gq, gk, gv = attn.attn_bwd(dq_, dk_, dv_, o, lse, ddo, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    say(f"  kernel {attn.attn_last_kernel()}")
    rq, rk, rv, _ = oracle.attention_backward(to_f64(q), to_f64(k), to_f64(v), to_f64(do), w.scale, w.causal)
    for name, got, ref in (("dQ", gq, rq), ("dK", gk, rk), ("dV", gv, rv)):
        g = to_f64(got)
        assert np.isfinite(g).all(), name
        err = float(np.abs(g - ref).max())
        say(f"  {name}: max|err|={err:.3e} max|ref|={float(np.abs(ref).max()):.3e} (tol {tol(ref):.3e})")
        assert err <= tol(ref), f"{name} error {err}"
    return gq, gk, gv


CASES = [
    # B, H, Tq, Tkv, causal
    (1, 2, 200, 200, False),
    (1, 2, 200, 200, True),
    (2, 3, 129, 129, True),
    (1, 1, 384, 384, True),
    (1, 2, 100, 300, True),     # bottom-right causal, Tq < Tkv
    (1, 2, 100, 300, False),
    (1, 1, 257, 1000, False),
    (1, 1, 33, 700, True),
    (1, 3, 5, 1, False),        # one key
    (1, 1, 2, 2, True),
    (1, 1, 300, 17, False),     # fewer keys than a key tile
    (2, 2, 64, 64, True),
    (1, 1, 1, 50, False),       # a single query
    (1, 2, 449, 449, True),     # 1-8 blocks per tile: every remainder of the unrolled loops
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,Tq,Tkv,causal", CASES)
def test_backward_shapes(B, H, Tq, Tkv, causal, d):
    check(Workload(f"bwd[{B},{H},{Tq},{Tkv},{'c' if causal else 'n'},d={d}]", B, H, Tq, Tkv, d, "bf16", causal,
                   seed=200 + Tq + Tkv + d))
    assert attn.attn_last_kernel().startswith(f"bwd_bf16_d{d}<")


# d = 64 grids with fewer than 768 128-wide tiles split each tile's serial
# loop over a pair of waves: query halves in dK/dV (decided by the key tiles),
# key halves in dQ (decided by the query tiles).  Each combination:
D64_PATH_CASES = [
    # B, H, Tq, Tkv, causal, dK/dV query halves, dQ key halves
    (8, 96, 129, 129, True, False, False),
    (8, 48, 300, 100, False, True, False),
    (8, 48, 100, 300, True, False, True),
    (2, 5, 333, 333, True, True, True),
]


@pytest.mark.parametrize("B,H,Tq,Tkv,causal,kvh,qh", D64_PATH_CASES)
def test_backward_d64_paths(B, H, Tq, Tkv, causal, kvh, qh):
    check(Workload(f"bwd[{B},{H},{Tq},{Tkv},{'c' if causal else 'n'},d=64]", B, H, Tq, Tkv, 64, "bf16", causal,
                   seed=300 + B * H + Tq))
    kern = attn.attn_last_kernel()
    assert ("query_halves=2" in kern) == kvh and ("key_halves=2" in kern) == qh, kern


def test_backward_long_head_full():
    """One 4096-token causal head: 64 query blocks through each pair of the
    small-grid dK/dV and dQ kernels, every gradient checked in full."""
    w = Workload("bwd_long_head", 1, 1, 4096, 4096, 64, "bf16", True, seed=41)
    check(w)
    kern = attn.attn_last_kernel()
    assert "query_halves=2" in kern and "key_halves=2" in kern, kern


def test_backward_gpt2_full():
    check(WORKLOADS["gpt2"])


def test_backward_gpt2_shape_d128_full():
    check(WORKLOADS["gpt2"].with_(name="gpt2_d128", d=128, seed=12))


def test_backward_spread_scores():
    check(Workload("bwd_k3", 1, 4, 512, 512, 64, "bf16", True, seed=9, k_factor=3.0))


def test_backward_deterministic():
    w = WORKLOADS["gpt2"].with_(B=1, H=4)
    q, k, v = (t.cuda() for t in make_qkv(w))
    do = upstream(w).cuda()
    o, lse = attn.attn_fwd(q, k, v, causal=True)
    a = attn.attn_bwd(q, k, v, o, lse, do, causal=True)
    b = attn.attn_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
