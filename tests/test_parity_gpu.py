"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Inputs are the seeded synthetic tensors of io_aware_exact_amd.inputs; the
oracle sees exactly the values uploaded (bf16-rounded for bf16 cases).
Tolerances: max-abs error on O <= 1e-5 for fp32 inputs and <= 2e-2 for bf16
inputs; max-abs error on LSE <= 1e-3.  Small cases compare every output.
The full-size prefill workloads compare every row of every head (mid-length,
full and causal), every row of one head plus sampled rows of two more (long),
or every row of four heads (head width 128), computed by the oracle in
chunks of query rows, in the same launch configuration the benchmark times;
the full-size decode workloads compare sampled heads.
"""

import math
import sys

import numpy as np
import pytest
import torch

import io_aware_exact_amd as attn
import oracle
from io_aware_exact_amd.inputs import WORKLOADS, Workload, make_qkv, to_f64

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

TOL_O = {"f32": 1e-5, "bf16": 2e-2}
TOL_LSE = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu(w: Workload, q, k, v, api=None):
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    if api == "decode" or (api is None and w.Tq == 1 and w.num_splits > 1):
        o, lse = attn.attn_decode(dq, dk, dv, scale=w.scale, num_splits=w.num_splits)
        lse = lse[:, :, None]
    elif w.dtype == "f32":
        o, lse = attn.attn_fwd_f32(dq, dk, dv, causal=w.causal, scale=w.scale)
    else:
        o, lse = attn.attn_fwd(dq, dk, dv, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return o, lse, attn.attn_last_kernel()


def compare(w: Workload, o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    eo = float(np.abs(to_f64(o_gpu) - o_ref).max())
    el = float(np.abs(to_f64(lse_gpu) - lse_ref).max())
    say(f"  {w.name}{what}: max|dO|={eo:.3e} (tol {TOL_O[w.dtype]}), max|dLSE|={el:.3e}")
    assert np.isfinite(to_f64(o_gpu)).all()
    assert eo <= TOL_O[w.dtype], f"O error {eo}"
    assert el <= TOL_LSE, f"LSE error {el}"
    return eo, el


def full_check(w: Workload, api=None):
    say(f"case {w}")
    q, k, v = make_qkv(w)
    o, lse, kern = run_gpu(w, q, k, v, api)
    say(f"  kernel {kern}")
    o_ref, lse_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), w.scale, w.causal)
    return compare(w, o, lse, o_ref, lse_ref)


# ------------------------------------------------------------ the named workloads

def test_tiny_fp32_full():
    full_check(WORKLOADS["tiny"])


def test_gpt2_bf16_causal_full():
    w = WORKLOADS["gpt2"]
    full_check(w)
    assert attn.attn_last_kernel().startswith("prefill_bf16_d64")


def _sampled_rows(T, n, rng):
    """First and last rows, rows around tile edges and a random spread."""
    edge = [0, 1, 31, 32, 63, 64, 127, 128, 129, T // 2, T - 129, T - 128, T - 2, T - 1]
    rnd = rng.choice(T, size=n, replace=False).tolist()
    return np.array(sorted(set(r for r in edge + rnd if 0 <= r < T)))


def _compare_head(w, q, k, v, o, lse, b, h, rows_per_chunk=4096):
    """Every row of head (b, h) against the oracle, in chunks of query rows
    (the causal mask uses each row's absolute index, so chunks are exact)."""
    og, lg = o[b, h].cpu(), lse[b, h].cpu()
    qb, kb, vb = to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h])
    eo = el = 0.0
    for r0 in range(0, w.Tq, rows_per_chunk):
        rows = np.arange(r0, min(w.Tq, r0 + rows_per_chunk))
        o_ref, lse_ref = oracle.attention(qb, kb, vb, w.scale, w.causal, rows=rows)
        eo = max(eo, float(np.abs(to_f64(og[r0:r0 + rows.size]) - o_ref).max()))
        el = max(el, float(np.abs(to_f64(lg[r0:r0 + rows.size]) - lse_ref).max()))
    assert np.isfinite(to_f64(og)).all()
    return eo, el


@pytest.mark.parametrize("name", ["mid", "mid_causal"])
def test_prefill_mid_every_head(name):
    """The mid-length prefill (2x16x4096, K x 3), full and causal: every row of
    every head, element by element, in the launch the benchmark times."""
    w = WORKLOADS[name]
    say(f"case {w} (every head, every row)")
    q, k, v = make_qkv(w)
    o, lse, kern = run_gpu(w, q, k, v)
    say(f"  kernel {kern}")
    worst_o = worst_l = 0.0
    for b in range(w.B):
        for h in range(w.H):
            eo, el = _compare_head(w, q, k, v, o, lse, b, h)
            worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
    say(f"  {w.B * w.H} heads x {w.Tq} rows: max|dO|={worst_o:.3e} (tol {TOL_O[w.dtype]}), max|dLSE|={worst_l:.3e}")
    assert worst_o <= TOL_O[w.dtype] and worst_l <= TOL_LSE


def test_prefill_long_full_head():
    """The long causal prefill (1x12x16384): every row of one head (in chunks
    of 2048 rows) and sampled rows of two more, element by element."""
    w = WORKLOADS["long"]
    say(f"case {w} (one full head, two sampled)")
    q, k, v = make_qkv(w)
    o, lse, kern = run_gpu(w, q, k, v)
    say(f"  kernel {kern}")
    eo, el = _compare_head(w, q, k, v, o, lse, 0, 7, rows_per_chunk=2048)
    say(f"  head 7, all {w.Tq} rows: max|dO|={eo:.3e}, max|dLSE|={el:.3e}")
    assert eo <= TOL_O[w.dtype] and el <= TOL_LSE
    rng = np.random.default_rng(1000 + w.seed)
    for b, h in [(0, 0), (0, w.H - 1)]:
        rows = _sampled_rows(w.Tq, 256, rng)
        o_ref, lse_ref = oracle.attention(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]), w.scale, w.causal,
                                          rows=rows)
        idx = torch.from_numpy(rows).cuda()
        compare(w, o[b, h][idx], lse[b, h][idx], o_ref, lse_ref, what=f"[b={b},h={h}, {rows.size} rows]")


def test_gpt2_shape_peaked_rows():
    """GPT-2-shaped causal prefill with K rows scaled by 4 (scores with a
    spread of 4 after scaling, so most rows are dominated by a few keys):
    every head, every row.  The largest error term is then the rounding of
    the dominant probability and of the output, each up to 2^-9 of |v|."""
    w = WORKLOADS["gpt2"].with_(name="gpt2_peaked", seed=11, k_factor=4.0)
    full_check(w)


@pytest.mark.parametrize("name", ["mid_d128", "mid_d128_causal"])
def test_prefill_d128_full_size(name):
    """The mid-length prefill at head width 128: every row of four heads."""
    w = WORKLOADS[name]
    say(f"case {w} (four full heads)")
    q, k, v = make_qkv(w)
    o, lse, kern = run_gpu(w, q, k, v)
    say(f"  kernel {kern}")
    for b, h in [(0, 0), (w.B - 1, w.H - 1), (0, 9), (1, 4)]:
        eo, el = _compare_head(w, q, k, v, o, lse, b, h)
        say(f"  [b={b},h={h}] max|dO|={eo:.3e}, max|dLSE|={el:.3e}")
        assert eo <= TOL_O[w.dtype] and el <= TOL_LSE


def test_decode_full_size_sampled():
    w = WORKLOADS["decode"]
    say(f"case {w} (sampled heads)")
    q, k, v = make_qkv(w)
    o, lse, kern = run_gpu(w, q, k, v)
    say(f"  kernel {kern}")
    assert "combine" in kern
    rng = np.random.default_rng(77)
    picks = [(0, 0), (w.B - 1, w.H - 1)] + [(int(b), int(h)) for b, h in
                                            zip(rng.integers(0, w.B, 14), rng.integers(0, w.H, 14))]
    for b, h in picks:
        o_ref, lse_ref = oracle.attention(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]), w.scale)
        compare(w, o[b, h], lse[b, h], o_ref, lse_ref, what=f"[b={b},h={h}]")
    # the split result against the unsplit kernel on the same inputs
    o1, lse1 = attn.attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=w.scale)
    torch.cuda.synchronize()
    d = float((o1.float() - o.float()).abs().max())
    say(f"  split vs unsplit max|dO|={d:.3e}")
    assert d <= 2e-2


# ------------------------------------------------------------ shapes and edges

PREFILL_CASES = [
    # B, H, Tq, Tkv, causal
    (1, 2, 200, 200, False),
    (1, 2, 200, 200, True),
    (2, 3, 129, 129, True),
    (1, 1, 384, 384, True),
    (1, 2, 100, 300, True),     # bottom-right causal, Tq < Tkv
    (1, 2, 100, 300, False),
    (1, 1, 257, 1000, False),
    (2, 2, 64, 64, True),
    (1, 1, 2, 2, True),
    (1, 3, 5, 1, False),        # one key
    (1, 1, 300, 17, False),     # fewer keys than a block
    (1, 1, 33, 700, True),
    (3, 1, 1000, 1000, True),
    (2, 4, 300, 300, False),    # B*H a multiple of 8, full: heads run one after another per XCD
    (1, 16, 257, 513, False),   # ... with Tq < Tkv and ragged ends
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,Tq,Tkv,causal", PREFILL_CASES)
def test_prefill_bf16_shapes(B, H, Tq, Tkv, causal, d):
    full_check(Workload(f"bf16[{B},{H},{Tq},{Tkv},{'c' if causal else 'n'},d={d}]", B, H, Tq, Tkv, d, "bf16",
                        causal, seed=11 + Tq + Tkv + d))
    if Tq > 1:
        assert attn.attn_last_kernel().startswith(f"prefill_bf16_d{d}<")


# d = 64 has three kernels: 128-row tiles; 64-row tiles whose key loop is
# split over two waves ("key_halves") when the 128-row tiles would number
# fewer than 768; and, for full attention, 256-row tiles of two 32-row
# sub-tiles per wave ("rows_per_wave=64") when their 512 resident tiles need
# fewer rounds than the 128-row kernel's 768.  All are exercised here with
# ragged ends and offsets; the key-halves cases with 48 heads also take its
# balanced (snake) unit order, one of them with a partial last round; the
# 256-row cases cover the head-major tile order (400 heads), the plain one
# (393 heads), T_q > T_kv and a partly empty last sub-tile (500 rows).
D64_PATH_CASES = [
    # B, H, Tq, Tkv, causal, key halves, 256-row tiles
    (8, 96, 129, 129, True, False, False),
    (8, 96, 100, 300, True, False, False),
    (4, 192, 200, 200, False, False, False),
    (4, 12, 1000, 1000, True, True, False),
    (2, 24, 1100, 1300, True, True, False),
    (3, 5, 333, 333, False, True, False),
    (1, 1, 65, 65, True, True, False),
    # 449 rows: tiles of 1-8 key blocks, so the unrolled loops end with every
    # remainder of unmasked and masked blocks
    (1, 192, 449, 449, True, False, False),
    (1, 192, 449, 449, False, False, False),
    (1, 2, 449, 449, True, True, False),
    (4, 100, 129, 200, False, False, True),
    (3, 131, 250, 77, False, False, True),
    (1, 200, 500, 500, False, False, True),
]


@pytest.mark.parametrize("B,H,Tq,Tkv,causal,halves,rows256", D64_PATH_CASES)
def test_prefill_bf16_d64_paths(B, H, Tq, Tkv, causal, halves, rows256):
    full_check(Workload(f"bf16[{B},{H},{Tq},{Tkv},{'c' if causal else 'n'},d=64]", B, H, Tq, Tkv, 64, "bf16",
                        causal, seed=3 + B * H + Tq))
    kern = attn.attn_last_kernel()
    assert ("key_halves=2" in kern) == halves, kern
    assert ("rows_per_wave=64" in kern) == rows256, kern


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("Tq,Tkv,causal", [(256, 256, False), (100, 100, True), (70, 333, True), (1, 65, False)])
def test_prefill_fp32_shapes(d, Tq, Tkv, causal):
    full_check(Workload(f"f32[d={d},{Tq},{Tkv},{'c' if causal else 'n'}]", 2, 2, Tq, Tkv, d, "f32", causal,
                        seed=5 + d + Tq))


SPLIT_CASES = [
    # B, H, Tq, Tkv, causal, kv_chunk
    (1, 2, 1000, 1000, True, 64),     # one block per unit
    (1, 2, 1000, 1000, True, 256),
    (2, 3, 129, 129, True, 64),       # ragged last tile
    (1, 2, 100, 300, True, 64),       # bottom-right causal, Tq < Tkv
    (1, 2, 100, 300, False, 128),
    (1, 1, 257, 1000, False, 192),    # chunk not a multiple of the block: rounded up
    (1, 1, 33, 700, True, 64),
    (3, 1, 1000, 1000, True, 0),      # automatic choice
    (1, 1, 300, 17, False, 64),       # one key block: nothing to split
    (1, 3, 5, 1, False, 64),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,Tq,Tkv,causal,chunk", SPLIT_CASES)
def test_prefill_split_shapes(B, H, Tq, Tkv, causal, chunk, d):
    w = Workload(f"split[{B},{H},{Tq},{Tkv},{'c' if causal else 'n'},kv={chunk},d={d}]", B, H, Tq, Tkv, d, "bf16",
                 causal, seed=60 + Tq + Tkv + d)
    say(f"case {w}")
    q, k, v = make_qkv(w)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o, lse = attn.attn_fwd_split(dq, dk, dv, causal=causal, scale=w.scale, kv_chunk=chunk)
    torch.cuda.synchronize()
    kern = attn.attn_last_kernel()
    say(f"  kernel {kern}")
    split = attn.attn_fwd_split_workspace_bytes(B, H, Tq, Tkv, d, causal, chunk) > 0
    assert ("combine" in kern) == split
    o_ref, lse_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), w.scale, causal)
    compare(w, o, lse, o_ref, lse_ref)
    o1, lse1 = attn.attn_fwd(dq, dk, dv, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    if not split:
        assert torch.equal(o, o1) and torch.equal(lse, lse1)


def test_gpt2_split_full():
    w = WORKLOADS["gpt2"]
    say(f"case {w} (split into 256-key units)")
    q, k, v = make_qkv(w)
    o, lse = attn.attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=w.scale, kv_chunk=256)
    torch.cuda.synchronize()
    kern = attn.attn_last_kernel()
    say(f"  kernel {kern}")
    assert "combine" in kern
    o_ref, lse_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), w.scale, True)
    compare(w, o, lse, o_ref, lse_ref)


@pytest.mark.parametrize("name", ["long_1head", "long_1head_full"])
def test_split_full_size_sampled(name):
    """A single 16K-key head: the automatic plan splits every long tile."""
    w = WORKLOADS[name]
    say(f"case {w} (automatic split, sampled rows)")
    q, k, v = make_qkv(w)
    o, lse = attn.attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    kern = attn.attn_last_kernel()
    say(f"  kernel {kern}")
    assert "combine" in kern
    rows = _sampled_rows(w.Tq, 64, np.random.default_rng(2000 + w.seed))
    o_ref, lse_ref = oracle.attention(to_f64(q[0, 0]), to_f64(k[0, 0]), to_f64(v[0, 0]), w.scale, w.causal,
                                      rows=rows)
    idx = torch.from_numpy(rows).cuda()
    compare(w, o[0, 0][idx], lse[0, 0][idx], o_ref, lse_ref, what=f"[{rows.size} rows]")


def test_fp32_scores_spread():
    w = WORKLOADS["tiny"].with_(name="tiny_k3", k_factor=3.0)
    full_check(w)


@pytest.mark.parametrize("B,H,Tkv,d,splits", [
    (2, 3, 1000, 128, 16), (3, 2, 77, 64, 3), (1, 1, 1, 128, 16), (4, 4, 8192, 64, 16),
    (2, 2, 512, 128, 1), (2, 2, 513, 128, 2), (1, 2, 40, 128, 45), (5, 3, 4097, 128, 7),
    (1, 12, 16384, 64, 0), (1, 32, 1000, 128, 0), (1, 2, 5000, 64, 64), (1, 1, 20000, 128, 129),
    (1, 4, 3000, 128, 0),       # automatic: 23 partitions (the minimum-keys cut of one per CU)
    (1, 8, 16384, 64, 0),       # automatic: 32 partitions, one workgroup per CU
])
def test_decode_shapes(B, H, Tkv, d, splits):
    full_check(Workload(f"decode[{B},{H},{Tkv},d={d},P={splits}]", B, H, 1, Tkv, d, "bf16", False,
                        seed=3 + Tkv, num_splits=splits), api="decode")
    used = splits if splits else attn.attn_decode_splits(B, H, H, Tkv, d)
    assert ("combine" in attn.attn_last_kernel()) == (min(used, Tkv) > 1)


def test_decode_batch1_full_size():
    """One sequence, 12 heads of 64, 16K cached keys: every head, automatic partitions."""
    full_check(WORKLOADS["decode_b1"], api="decode")
    assert "combine" in attn.attn_last_kernel()


def gqa_check(w: Workload):
    say(f"case {w}")
    q, k, v = make_qkv(w)
    o, lse = attn.attn_decode_gqa(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, num_splits=w.num_splits)
    torch.cuda.synchronize()
    kern = attn.attn_last_kernel()
    say(f"  kernel {kern}")
    o_ref, lse_ref = oracle.attention_gqa(to_f64(q), to_f64(k), to_f64(v), w.scale)
    compare(w, o, lse[:, :, None], o_ref, lse_ref)
    return kern


@pytest.mark.parametrize("B,Hq,Hkv,Tkv,d,splits", [
    (2, 8, 8, 700, 128, 4),      # one query head per group: attn_decode's case
    (2, 8, 4, 700, 128, 4),      # groups of 2
    (2, 8, 2, 1000, 128, 16),    # groups of 4
    (2, 8, 1, 1000, 128, 7),     # multi-query: one key/value head
    (1, 16, 2, 513, 128, 1),     # groups of 8, unsplit
    (3, 6, 2, 301, 64, 5),       # groups of 3 (head tile 1)
    (2, 12, 2, 257, 64, 3),      # groups of 6 (head tile 2)
    (1, 32, 2, 90, 64, 200),     # groups of 16 (two tiles of 8), splits clamped to Tkv
    (1, 4, 1, 1, 128, 16),       # a single cached key
    (2, 8, 2, 3000, 128, 0),     # automatic partitions
    (1, 64, 1, 700, 128, 5),     # groups of 64: two 32-head tiles per kv head (matrix-core kernel)
    (2, 8, 2, 777, 64, 0),       # groups of 4 at d = 64, automatic partitions
    (2, 40, 1, 333, 64, 3),      # groups of 40: a partial second tile
    (3, 16, 2, 1, 64, 4),        # groups of 8 against a single key
    (1, 32, 4, 5000, 128, 0),    # groups of 8, automatic partitions
])
def test_gqa_decode_shapes(B, Hq, Hkv, Tkv, d, splits):
    kern = gqa_check(Workload(f"gqa[{B},{Hq}/{Hkv},{Tkv},d={d},P={splits}]", B, Hq, 1, Tkv, d, "bf16", False,
                              seed=40 + Hq + Tkv, num_splits=splits, Hkv=Hkv))
    used = splits if splits else attn.attn_decode_splits(B, Hq, Hkv, Tkv, d)
    assert ("combine" in kern) == (min(used, Tkv) > 1)
    assert kern.startswith("decode_mfma") == (Hq // Hkv >= 4)


def test_gqa_decode_full_size_sampled():
    w = WORKLOADS["decode_gqa"]
    say(f"case {w} (sampled heads)")
    q, k, v = make_qkv(w)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o, lse = attn.attn_decode_gqa(dq, dk, dv, scale=w.scale, num_splits=w.num_splits)
    torch.cuda.synchronize()
    say(f"  kernel {attn.attn_last_kernel()}")
    G = w.H // w.kv_heads
    rng = np.random.default_rng(78)
    picks = [(0, 0), (w.B - 1, w.H - 1)] + [(int(b), int(h)) for b, h in
                                            zip(rng.integers(0, w.B, 14), rng.integers(0, w.H, 14))]
    for b, h in picks:
        o_ref, lse_ref = oracle.attention(to_f64(q[b, h]), to_f64(k[b, h // G]), to_f64(v[b, h // G]), w.scale)
        compare(w, o[b, h], lse[b, h], o_ref, lse_ref, what=f"[b={b},h={h}]")
    # against the multi-head kernel on key/value heads repeated G times
    kr = dk.repeat_interleave(G, dim=1).contiguous()
    vr = dv.repeat_interleave(G, dim=1).contiguous()
    o1, lse1 = attn.attn_decode(dq, kr, vr, scale=w.scale, num_splits=w.num_splits)
    torch.cuda.synchronize()
    dO = float((o1.float() - o.float()).abs().max())
    dL = float((lse1 - lse).abs().max())
    say(f"  grouped vs repeated heads max|dO|={dO:.3e} max|dLSE|={dL:.3e}")
    assert dO <= 2e-2 and dL <= TOL_LSE


@pytest.mark.parametrize("d", [64, 128])
def test_single_query_through_attn_fwd(d):
    w = Workload(f"fwd_tq1[d={d}]", 3, 4, 1, 2049, d, "bf16", True, seed=21)
    full_check(w)
    assert attn.attn_last_kernel().startswith("decode_bf16")


def test_spread_scores_bf16():
    w = Workload("bf16_k3", 1, 4, 512, 512, 64, "bf16", False, seed=8, k_factor=3.0)
    full_check(w)
    full_check(w.with_(causal=True, name="bf16_k3_causal"))


# one shape per forward kernel: key halves, 128-row causal, 256-row full
# attention, head width 128, and a single query (the decode kernel)
LSE_OPTIONAL_CASES = [
    (1, 2, 130, 130, 64, True, "key_halves=2"),
    (8, 96, 129, 129, 64, True, "bq=128"),
    (4, 100, 129, 200, 64, False, "rows_per_wave=64"),
    (1, 3, 200, 200, 128, False, "prefill_bf16_d128"),
    (2, 3, 1, 300, 64, True, "decode_bf16"),
]


@pytest.mark.parametrize("B,H,Tq,Tkv,d,causal,kern", LSE_OPTIONAL_CASES)
def test_lse_optional_and_outputs_in_place(B, H, Tq, Tkv, d, causal, kern):
    """Without an LSE pointer the kernel writes O alone, bitwise equal to the
    call that also writes the LSE, into the caller's buffer."""
    w = Workload("inplace", B, H, Tq, Tkv, d, "bf16", causal, seed=4)
    q, k, v = [t.cuda() for t in make_qkv(w)]
    o_ref, lse_ref = attn.attn_fwd(q, k, v, causal=causal)
    out = torch.full_like(q, float("nan"))
    o2 = attn.attn_fwd(q, k, v, causal=causal, out=out, return_lse=False)
    torch.cuda.synchronize()
    assert kern in attn.attn_last_kernel(), attn.attn_last_kernel()
    assert o2.data_ptr() == out.data_ptr()
    assert torch.equal(o2, o_ref)


@pytest.mark.parametrize("B,H,T,causal", [(1, 4, 1024, True), (4, 100, 129, False), (8, 96, 129, True)])
def test_deterministic_across_runs(B, H, T, causal):
    """Bitwise equal results from two calls (no atomics, no order that
    depends on timing), on the key-halves, 256-row and 128-row kernels."""
    w = WORKLOADS["gpt2"].with_(B=B, H=H, Tq=T, Tkv=T, causal=causal)
    q, k, v = [t.cuda() for t in make_qkv(w)]
    o1, l1 = attn.attn_fwd(q, k, v, causal=causal)
    o2, l2 = attn.attn_fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_misaligned_view_rejected_before_launch():
    base = torch.zeros(1 * 1 * 64 * 64 + 1, dtype=torch.bfloat16, device="cuda")
    q = base[1:].view(1, 1, 64, 64)
    k = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="aligned"):
        attn.attn_fwd(q, k, k)


def test_wrong_output_shapes_rejected_before_launch():
    """Outputs the caller passes must have exactly the shape the call writes;
    a smaller buffer is refused in the binding, before any launch."""
    q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16, device="cuda")
    o_small = torch.empty(1, 2, 63, 64, dtype=torch.bfloat16, device="cuda")
    lse_small = torch.empty(1, 2, 63, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="o must have shape"):
        attn.attn_fwd(q, q, q, out=o_small)
    with pytest.raises(ValueError, match="lse must have shape"):
        attn.attn_fwd(q, q, q, lse=lse_small)
    with pytest.raises(ValueError, match="o must have shape"):
        attn.prepared_fwd(q, q, q, o_small, None, False)
    with pytest.raises(ValueError, match="o must have shape"):
        attn.attn_fwd_f32(q.float(), q.float(), q.float(), out=o_small.float())
    lse = torch.empty(1, 2, 64, dtype=torch.float32, device="cuda")
    d_small = torch.empty(1, 2, 64, 32, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="dk must have shape"):
        attn.attn_bwd(q, q, q, q, lse, q, dk=d_small)
    with pytest.raises(ValueError, match="lse must have shape"):
        attn.attn_bwd(q, q, q, q, lse_small, q)
    qd = torch.zeros(2, 4, 1, 64, dtype=torch.bfloat16, device="cuda")
    kd = torch.zeros(2, 4, 100, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="lse must have shape"):
        attn.attn_decode(qd, kd, kd, lse=torch.empty(2, 3, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="workspace must be a GPU tensor"):
        attn.attn_decode(qd, kd, kd, num_splits=4, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    torch.cuda.synchronize()


def test_no_device_allocation_during_call():
    """The score matrix never exists: a prefill call allocates nothing on the
    device beyond the caller's O and LSE (the library has no allocator)."""
    w = WORKLOADS["long"].with_(H=2)
    q, k, v = [t.cuda() for t in make_qkv(w)]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    attn.attn_fwd(q, k, v, causal=True, out=o, lse=lse)   # the runtime's one-time set-up of a first launch
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    attn.attn_fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    # one T x T fp32 score matrix per head would be 1 GiB here
    assert free0 - free1 < (1 << 20)


def test_prepared_calls_allocate_nothing():
    """With outputs and workspaces preallocated, the split forward, grouped
    decode and backward calls allocate no device memory."""
    w = WORKLOADS["long_1head"].with_(Tq=4096, Tkv=4096)
    q, k, v = [t.cuda() for t in make_qkv(w)]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    ws = torch.empty(attn.attn_fwd_split_workspace_bytes(1, 1, 4096, 4096, 64, True, 0), dtype=torch.uint8,
                     device="cuda")
    fwd = attn.prepared_fwd(q, k, v, o, lse, True, kv_chunk=0, workspace=ws)
    dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dk, dv = torch.empty_like(dq), torch.empty_like(dq)
    bws = torch.empty(attn.attn_bwd_workspace_bytes(1, 1, 4096), dtype=torch.uint8, device="cuda")
    do = torch.ones_like(q)
    bwd = attn.prepared_bwd(q, k, v, o, lse, do, dq, dk, dv, True, bws)
    g = Workload("gqa_alloc", 2, 16, 1, 4096, 128, "bf16", False, seed=31, Hkv=2)
    gq, gk, gv = [t.cuda() for t in make_qkv(g)]
    go = torch.empty_like(gq)
    glse = torch.empty((2, 16), dtype=torch.float32, device="cuda")
    gws = torch.empty(attn.attn_decode_workspace_bytes(2, 16, 128, 8), dtype=torch.uint8, device="cuda")
    dec = attn.prepared_decode(gq, gk, gv, go, glse, 8, gws)
    fwd(); bwd(); dec()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        fwd(); bwd(); dec()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free0 - free1 < (1 << 20)


def test_calls_run_on_the_current_stream():
    """Every entry point enqueues on the caller's stream: results computed on a
    side stream (default priority) equal the default stream's."""
    w = Workload("streams", 2, 3, 300, 300, 64, "bf16", True, seed=32)
    q, k, v = [t.cuda() for t in make_qkv(w)]
    do = torch.ones_like(q)
    ref_o, ref_l = attn.attn_fwd(q, k, v, causal=True)
    ref_g = attn.attn_bwd(q, k, v, ref_o, ref_l, do, causal=True)
    ref_d = attn.attn_decode(q[:, :, :1].contiguous(), k, v, num_splits=4)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        o, l = attn.attn_fwd(q, k, v, causal=True)
        g = attn.attn_bwd(q, k, v, o, l, do, causal=True)
        d = attn.attn_decode(q[:, :, :1].contiguous(), k, v, num_splits=4)
    side.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
    for a, b in zip(g, ref_g):
        assert torch.equal(a, b)
    assert torch.equal(d[0], ref_d[0]) and torch.equal(d[1], ref_d[1])



@pytest.mark.parametrize("api,d", [("decode", 128), ("prefill_split", 128), ("prefill", 128), ("prefill", 64)])
def test_longest_accepted_head(api, d):
    """One head of the most keys the 32-bit buffer ranges accept (K and V
    2 GiB each: 8,388,607 keys at d = 128, 16,777,215 at d = 64), sampled rows
    against the oracle: the oracle runs on 2^20-key partitions and merges them
    with its own partition combine."""
    T = (1 << 31) // (2 * d) - 1
    g = torch.Generator(device="cuda").manual_seed(77)
    k = torch.randn((1, 1, T, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((1, 1, T, d), generator=g, device="cuda").to(torch.bfloat16)
    tq = 1 if api == "decode" else 130
    q = torch.randn((1, 1, tq, d), generator=g, device="cuda").to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    say(f"case {api}: T_kv={T}, T_q={tq}, d={d}")
    if api == "decode":
        o, lse = attn.attn_decode(q, k, v, scale=scale, num_splits=0)
        lse = lse[:, :, None]
    elif api == "prefill_split":
        o, lse = attn.attn_fwd_split(q, k, v, causal=False, scale=scale, kv_chunk=0)
    else:
        o, lse = attn.attn_fwd(q, k, v, causal=False, scale=scale)
    torch.cuda.synchronize()
    say(f"  kernel {attn.attn_last_kernel()}")
    if api == "prefill":
        assert ("key_halves=2" in attn.attn_last_kernel()) == (d == 64)
    rows = sorted({0, tq - 1})
    qr = to_f64(q[:, :, rows])
    kh, vh = k.cpu(), v.cpu()
    parts = [oracle.attention(qr, to_f64(kh[:, :, i:i + (1 << 20)]), to_f64(vh[:, :, i:i + (1 << 20)]), scale)
             for i in range(0, T, 1 << 20)]
    o_ref, lse_ref = oracle.combine_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    eo = float(np.abs(to_f64(o[:, :, rows]) - o_ref).max())
    el = float(np.abs(to_f64(lse[:, :, rows]) - lse_ref).max())
    say(f"  max|dO|={eo:.2e} max|dLSE|={el:.2e}")
    assert eo <= 2e-2 and el <= 1e-3
