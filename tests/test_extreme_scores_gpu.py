"""Score rows far wider than the exponent range, through every forward kernel.

Each head's scores follow one pattern over the key axis, spanning about
+-600 in natural units (about +-865 in base 2, where 2^x overflows fp32
past 128):
  rising      - the largest scores come last, so every block raises the
                running maximum and the block's exponentials against the old
                reference are infinite: the kernels must detect the
                non-finite block sum and rescale;
  falling     - block 0 holds the maximum, later terms underflow to 0;
  late spike  - flat low scores with one key far above them near the end;
  alternating - signs alternate and magnitudes grow along the keys.
q is +-1 in every component and each key is one bf16 value r_j repeated over
d, so s_ij = scale * d * q_i * r_j and every dot product is exact in fp32 (a
sum of up to 128 copies of an 8-bit significand).  Both sides see the same
bf16 (or fp32) inputs; the oracle is the float64 definition.
"""

import math
import sys

import numpy as np
import pytest
import torch

import io_aware_exact_amd as attn
import oracle
from io_aware_exact_amd.inputs import make_tensor, to_f64
from test_sweep_gpu import float32_definition_error


def gpu(fn):
    """Mark a case that runs kernels (the host check below runs anywhere)."""
    fn = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")(fn)
    return pytest.mark.gpu(fn)


TOL_O_F32 = 1e-5
TOL_LSE = 1e-3
SPAN = 600.0        # largest |score| in natural units
PATTERNS = ["rising", "falling", "late spike", "alternating"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def key_values(pattern, Tkv, R):
    """r_j for one head (before the bf16 rounding)."""
    j = np.arange(Tkv, dtype=np.float64)
    x = 2.0 * j / max(Tkv - 1, 1) - 1.0                       # -1 .. 1
    if pattern == "rising":
        return R * x
    if pattern == "falling":
        return -R * x
    if pattern == "late spike":
        r = np.full(Tkv, -0.25 * R)
        r[Tkv - 1 - Tkv // 7] = R
        return r
    if pattern == "alternating":
        return R * np.where(j % 2 == 0, 1.0, -1.0) * (j + 1) / Tkv
    raise ValueError(pattern)


def extreme_qkv(B, H, Hkv, Tq, Tkv, d, scale, dtype, seed):
    """q = +-1 rows, k rows = r_j * ones(d) with K/V head h of batch b taking
    pattern (h + b) mod 4, v seeded normal.  Every third query row has the
    sign -1, so that both a pattern and its mirror image are seen."""
    R = SPAN / (scale * d)
    k = np.empty((B, Hkv, Tkv, d))
    for b in range(B):
        for h in range(Hkv):
            r = key_values(PATTERNS[(h + b) % 4], Tkv, R)
            k[b, h] = r[:, None]
    sign = np.where(np.arange(Tq) % 3 == 2, -1.0, 1.0)
    q = np.broadcast_to(sign[None, None, :, None], (B, H, Tq, d)).copy()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    # both kernels get bf16-representable key values, so the fp32 sums are exact
    kt = torch.from_numpy(k).to(torch.bfloat16).to(tdt).contiguous()
    qt = torch.from_numpy(q).to(tdt).contiguous()
    vt = make_tensor(seed, "v", B, Hkv, Tkv, d, dtype)
    return qt, kt, vt


def check(o, lse, q, k, v, scale, causal, dtype, gqa=False):
    torch.cuda.synchronize()
    ref = oracle.attention_gqa if gqa else oracle.attention
    qd, kd, vd = to_f64(q), to_f64(k), to_f64(v)
    o_ref, lse_ref = ref(qd, kd, vd, scale, causal)
    g = to_f64(o)
    assert np.isfinite(g).all(), "non-finite output"
    err = np.abs(g - o_ref)
    el = float(np.abs(to_f64(lse).reshape(lse_ref.shape) - lse_ref).max())   # decode's LSE is [B, H]
    say(f"  {attn.attn_last_kernel()}: max|dO| {err.max():.3e} max|dLSE| {el:.3e} "
        f"(LSE range {lse_ref.min():.1f} .. {lse_ref.max():.1f})")
    if dtype == "bf16":
        # two bf16 roundings (P and O) at unit roundoff 2^-8, as for every bf16 case
        a_ref, _ = ref(qd, kd, np.abs(vd), scale, causal)
        bound = 2.0 ** -8 * (np.abs(o_ref) + a_ref) * (1 + 2.0 ** -6)
        assert float((err / bound).max()) <= 1.0, f"O error {err.max()}"
    else:
        # at |s| near 600 the fp32 rounding of s * scale alone moves P by ~3e-5
        # relative: the bar is the larger of 1e-5 and twice the error of the
        # definition itself evaluated in float32
        tol = max(TOL_O_F32, 2.0 * float32_definition_error(q, k, v, scale, causal, o_ref))
        assert float(err.max()) <= tol, f"O error {err.max()} (bar {tol:.3e})"
    assert el <= TOL_LSE, f"LSE error {el}"


PREFILL = [  # B, H, Tq, Tkv, d, causal -- small grids take the key-halves kernel at d = 64
    (1, 4, 300, 300, 64, False),
    (1, 4, 300, 300, 64, True),
    (2, 4, 1000, 1000, 64, True),
    (1, 4, 70, 513, 64, True),
    (1, 4, 129, 700, 64, False),
    (1, 96, 1024, 1024, 64, True),      # 768 tiles of 128 rows: the 128-row kernel
    (1, 96, 1024, 1024, 64, False),
    (4, 100, 129, 200, 64, False),      # 800 tiles of 128 rows, 400 of 256: the 256-row kernel
    (1, 4, 300, 300, 128, False),
    (2, 4, 1000, 1000, 128, True),
    (1, 4, 70, 513, 128, True),
]


@gpu
@pytest.mark.parametrize("B,H,Tq,Tkv,d,causal", PREFILL)
def test_extreme_prefill_bf16(B, H, Tq, Tkv, d, causal):
    scale = d ** -0.5
    say(f"case extreme prefill bf16 B={B} H={H} Tq={Tq} Tkv={Tkv} d={d} causal={causal}")
    q, k, v = extreme_qkv(B, H, H, Tq, Tkv, d, scale, "bf16", 40)
    o, lse = attn.attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    check(o, lse, q, k, v, scale, causal, "bf16")


@gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_extreme_split_prefill(d, causal):
    B, H, T = 1, 4, 2000
    scale = d ** -0.5
    say(f"case extreme split prefill B={B} H={H} T={T} d={d} causal={causal} kv_chunk=256")
    q, k, v = extreme_qkv(B, H, H, T, T, d, scale, "bf16", 41)
    o, lse = attn.attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, kv_chunk=256)
    assert "kv_chunk" in attn.attn_last_kernel()
    check(o, lse, q, k, v, scale, causal, "bf16")


@gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits", [1, 7, 16])
def test_extreme_decode(d, splits):
    B, H, Tkv = 3, 8, 3000
    scale = d ** -0.5
    say(f"case extreme decode B={B} H={H} Tkv={Tkv} d={d} splits={splits}")
    q, k, v = extreme_qkv(B, H, H, 1, Tkv, d, scale, "bf16", 42)
    o, lse = attn.attn_decode(q.cuda(), k.cuda(), v.cuda(), scale=scale, num_splits=splits)
    check(o, lse, q, k, v, scale, False, "bf16")


@gpu
@pytest.mark.parametrize("splits", [1, 16])
def test_extreme_gqa_decode(splits):
    B, Hq, Hkv, Tkv, d = 2, 32, 8, 3000, 128
    scale = d ** -0.5
    say(f"case extreme grouped decode B={B} Hq={Hq} Hkv={Hkv} Tkv={Tkv} d={d} splits={splits}")
    q, k, v = extreme_qkv(B, Hq, Hkv, 1, Tkv, d, scale, "bf16", 43)
    o, lse = attn.attn_decode_gqa(q.cuda(), k.cuda(), v.cuda(), scale=scale, num_splits=splits)
    check(o, lse, q, k, v, scale, False, "bf16", gqa=True)


@gpu
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_extreme_fp32(d, causal):
    B, H, T = 1, 4, 300
    scale = d ** -0.5
    say(f"case extreme fp32 B={B} H={H} T={T} d={d} causal={causal}")
    q, k, v = extreme_qkv(B, H, H, T, T, d, scale, "f32", 44)
    o, lse = attn.attn_fwd_f32(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    check(o, lse, q, k, v, scale, causal, "f32")


def test_patterns_span_past_the_exponent_range():
    """The inputs really do what the cases above rely on (host only): scores
    reach +-SPAN, and a rising row's later block overflows 2^x against
    block 0's maximum."""
    d, scale, Tkv = 64, 0.125, 300
    q, k, _ = extreme_qkv(1, 4, 4, 2, Tkv, d, scale, "bf16", 45)
    s = np.einsum("hd,htd->ht", to_f64(q)[0, :, 0], to_f64(k)[0]) * scale    # (H, Tkv), query row 0
    assert abs(np.abs(s).max() - SPAN) < 0.01 * SPAN
    rising = s[0]
    assert (rising[-64:].max() - rising[:64].max()) / math.log(2.0) > 128


@gpu
@pytest.mark.parametrize("B,H,Tq,Tkv,d,causal", [
    (1, 4, 300, 300, 64, False), (1, 4, 300, 300, 64, True), (2, 4, 1000, 1000, 64, True),
    (1, 4, 300, 300, 128, False), (1, 4, 257, 400, 128, True)])
def test_extreme_backward(B, H, Tq, Tkv, d, causal):
    """The backward takes O and LSE as inputs: both sides get the GPU forward's
    bf16 O and fp32 LSE (|LSE| up to 600), so P = exp(s * scale - LSE) is
    recomputed from the same numbers.

    Bar, per element: |g_gpu - g| <= 2^-8 (|g| + A) (1 + 2^-6) + E + 1e-6 max|g|.
    The kernels round P (for dV) and dS = P (dP - D) (for dQ and dK) to bf16,
    2^-9 relative per term; A sums the terms of each product in absolute
    value: scale |dS| |K| for dQ, scale |dS|^T |Q| for dK, |P|^T |dO| for dV.
    E carries the fp32 error of dP - D, which two different summations of d
    products form (a d-term sum errs by at most d 2^-24 sum|terms|), through
    the same products: scale (P e) |K| for dQ, scale (P e)^T |Q| for dK.
    Where P is one-hot and O is that key's V, dP - D is 0 exactly and only
    this residue remains.  With |k| up to 75 here, dQ sums large terms that
    nearly cancel, which a bar relative to max|dQ| (the ordinary backward
    cases') does not cover."""
    scale = d ** -0.5
    say(f"case extreme backward B={B} H={H} Tq={Tq} Tkv={Tkv} d={d} causal={causal}")
    q, k, v = extreme_qkv(B, H, H, Tq, Tkv, d, scale, "bf16", 46)
    do = make_tensor(47, "v", B, H, Tq, d, "bf16")
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = attn.attn_fwd(qc, kc, vc, causal=causal, scale=scale)
    gq, gk, gv = attn.attn_bwd(qc, kc, vc, o, lse, doc, causal=causal, scale=scale)
    torch.cuda.synchronize()
    say(f"  {attn.attn_last_kernel()}")
    Q, K, V, O, dO, L = (to_f64(t) for t in (q, k, v, o, do, lse))
    refs = oracle.attention_backward_from_lse(Q, K, V, O, dO, L, scale, causal)
    # magnitudes of the terms each gradient sums (for the rounding bound only)
    s_ = scale * (Q @ np.swapaxes(K, -1, -2))
    if causal:
        s_ = np.where(np.arange(Tkv)[None, :] > np.arange(Tq)[:, None] + (Tkv - Tq), -np.inf, s_)
    P = np.exp(s_ - L[..., None])
    dS = P * (dO @ np.swapaxes(V, -1, -2) - (dO * O).sum(-1)[..., None])
    e32 = d * 2.0 ** -24 * (np.abs(dO) @ np.swapaxes(np.abs(V), -1, -2) + (np.abs(dO) * np.abs(O)).sum(-1)[..., None])
    Pe = P * e32
    A = {"dQ": scale * (np.abs(dS) @ np.abs(K)), "dK": scale * (np.swapaxes(np.abs(dS), -1, -2) @ np.abs(Q)),
         "dV": np.swapaxes(P, -1, -2) @ np.abs(dO)}
    E = {"dQ": scale * (Pe @ np.abs(K)), "dK": scale * (np.swapaxes(Pe, -1, -2) @ np.abs(Q)), "dV": 0.0}
    for name, got, ref in zip(("dQ", "dK", "dV"), (gq, gk, gv), refs[:3]):
        g = to_f64(got)
        assert np.isfinite(g).all(), name
        err = np.abs(g - ref)
        bound = 2.0 ** -8 * (np.abs(ref) + A[name]) * (1 + 2.0 ** -6) + E[name] + 1e-6 * float(np.abs(ref).max())
        ratio = float((err / bound).max())
        say(f"  {name}: max|err| {err.max():.3e} max|ref| {float(np.abs(ref).max()):.3e} max err/bound {ratio:.3f}")
        assert ratio <= 1.0, f"{name} error {err.max()} (err/bound {ratio})"
