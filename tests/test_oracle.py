"""Pins of the float64 oracle against what the pages and the mathematics fix.

Nothing here touches a GPU or the HIP library.  Each check ties the oracle to
something other than itself: the worked example printed on "E8.1 IO-aware
attention", closed forms, invariants, special cases, brute force in plain
Python loops on tiny inputs, and PyTorch's CPU attention in float64.

``PIN_CHECKS`` below is also run against deliberately broken copies of the
oracle (a dropped scale, transposed operands, a softmax over the wrong axis,
a flipped causal mask, ...) to show that each plausible mistake is caught;
``MORE_MUTANTS`` does the same for the blockwise recurrence, the one-query
online form, the partition merge, the split and the grouped-query mapping.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- worked example

def test_worked_example_after_block_1():
    g = _load("online_softmax_worked_example.json")
    states = oracle.online_softmax_states(g["scores"], g["block"])
    m1, l1 = states[0]
    assert m1 == g["after_block_1"]["m"]
    half_ulp = 0.5 * 10 ** (-g["after_block_1"]["printed_decimals"])
    assert abs(l1 - g["after_block_1"]["l"]) <= half_ulp


def test_worked_example_final_state_equals_full_row():
    g = _load("online_softmax_worked_example.json")
    s = g["scores"]
    m, l = oracle.online_softmax_states(s, g["block"])[-1]
    assert m == max(s)
    assert l == pytest.approx(math.fsum(math.exp(x - max(s)) for x in s), rel=1e-14)
    # the same row as a d=1 attention problem: q=[1], k_j=[s_j], scale 1
    q = np.ones((1, 1))
    k = np.array(s, dtype=np.float64)[:, None]
    v = np.eye(len(s))[:, :3]
    _, lse = attention(q, k, v, scale=1.0)
    assert lse[0] == pytest.approx(m + math.log(l), rel=1e-14)


def test_worked_example_split_into_its_two_blocks():
    """The two printed blocks merged by the cross-partition rescaling give the
    full row (the split form of the same recurrence)."""
    g = _load("online_softmax_worked_example.json")
    s = np.array(g["scores"], dtype=np.float64)
    q = np.ones((1, 1))
    k = s[:, None]
    rng = np.random.default_rng(7)
    v = rng.standard_normal((len(s), 5))
    o_full, lse_full = attention(q, k, v, 1.0)
    o_split, lse_split = oracle.split_attention(q, k, v, 1.0, num_splits=2)
    np.testing.assert_allclose(o_split, o_full, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse_split, lse_full, rtol=1e-14)
    # block 1's normaliser is the printed state
    m1, l1 = oracle.online_softmax_states(s, 4)[0]
    _, lse_b1 = attention(q, k[:4], v[:4], 1.0)
    assert lse_b1[0] == pytest.approx(m1 + math.log(l1), rel=1e-14)


# ---------------------------------------------------------------- blockwise == full

@pytest.mark.parametrize("n", [1, 2, 7, 17, 64])
def test_blockwise_equals_full_for_every_block_size(n):
    rng = np.random.default_rng(100 + n)
    d, dv = 5, 4
    q = _rand(rng, d)
    K = 3.0 * _rand(rng, n, d)
    V = _rand(rng, n, dv)
    ref = oracle.standard_attention(q, K, V)
    o_def, _ = attention(q[None], K, V, scale=1.0 / math.sqrt(d))
    np.testing.assert_allclose(o_def[0], ref, rtol=1e-12, atol=1e-13)
    for block in range(1, n + 1):
        got = oracle.online_attention(q, K, V, block)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    s = (K @ q) / math.sqrt(d)
    for block in range(1, n + 1):
        m, l = oracle.online_softmax_states(s, block)[-1]
        assert m == s.max()
        assert l == pytest.approx(math.fsum(math.exp(x - s.max()) for x in s), rel=1e-12)


@pytest.mark.parametrize("bad", [0, -1, -64])
def test_block_below_one_raises(bad):
    rng = np.random.default_rng(1)
    with pytest.raises(ValueError):
        oracle.online_attention(_rand(rng, 4), _rand(rng, 3, 4), _rand(rng, 3, 2), bad)
    with pytest.raises(ValueError):
        oracle.online_softmax_states([1.0, 2.0], bad)
    with pytest.raises(ValueError):
        oracle.num_blocks(10, bad)


# ---------------------------------------------------------------- pin suite

def _brute(q, k, v, scale, causal):
    """The definition in plain Python loops (math.exp, fsum): no numpy
    arithmetic, so it cannot share a mistake with the oracle's matmuls."""
    q = np.asarray(q).tolist()
    k = np.asarray(k).tolist()
    v = np.asarray(v).tolist()
    tq, tkv, dv = len(q), len(k), len(v[0])
    o, lse = [], []
    for i in range(tq):
        s = []
        for j in range(tkv):
            if causal and j > i + (tkv - tq):
                continue
            s.append((j, scale * math.fsum(a * b for a, b in zip(q[i], k[j]))))
        mx = max(x for _, x in s)
        w = [(j, math.exp(x - mx)) for j, x in s]
        den = math.fsum(x for _, x in w)
        o.append([math.fsum(x * v[j][c] for j, x in w) / den for c in range(dv)])
        lse.append(mx + math.log(den))
    return np.array(o), np.array(lse)


def _pin_tkv1(fn):
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 6, 4), _rand(rng, 1, 4), _rand(rng, 1, 3)
    o, lse = fn(q, k, v, 0.7, False)
    ok = np.allclose(o, np.repeat(v, 6, axis=0), rtol=0, atol=1e-15)
    return ok and np.allclose(lse, 0.7 * (q @ k[0]), rtol=1e-14, atol=1e-15)


def _pin_zero_query(fn):
    rng = np.random.default_rng(12)
    q, k, v = np.zeros((3, 4)), _rand(rng, 9, 4), _rand(rng, 9, 5)
    o, lse = fn(q, k, v, 0.5, False)
    return np.allclose(o, v.mean(axis=0)[None], atol=1e-14) and np.allclose(lse, math.log(9), atol=1e-14)


def _pin_ones_value(fn):
    rng = np.random.default_rng(13)
    q, k = _rand(rng, 5, 4), 2.0 * _rand(rng, 8, 4)
    o, _ = fn(q, k, np.ones((8, 3)), 0.5, False)
    o_c, _ = fn(q, k, np.ones((8, 3)), 0.5, True)
    return np.allclose(o, 1.0, atol=1e-14) and np.allclose(o_c, 1.0, atol=1e-14)


def _pin_causal_row0(fn):
    rng = np.random.default_rng(14)
    q, k, v = _rand(rng, 6, 4), _rand(rng, 6, 4), _rand(rng, 6, 3)
    o, lse = fn(q, k, v, 0.5, True)
    return np.allclose(o[0], v[0], atol=1e-15) and abs(lse[0] - 0.5 * q[0] @ k[0]) < 1e-14


def _pin_two_keys(fn):
    """T_kv = 2 has the closed form O = sigmoid(s0 - s1) v0 + sigmoid(s1 - s0) v1,
    lse = max + log1p(exp(-|s0 - s1|))."""
    rng = np.random.default_rng(15)
    q, k, v = _rand(rng, 4, 3), _rand(rng, 2, 3), _rand(rng, 2, 2)
    o, lse = fn(q, k, v, 0.9, False)
    s0, s1 = 0.9 * (q @ k[0]), 0.9 * (q @ k[1])
    a = 1.0 / (1.0 + np.exp(s1 - s0))
    o_ref = a[:, None] * v[0][None] + (1 - a)[:, None] * v[1][None]
    lse_ref = np.maximum(s0, s1) + np.log1p(np.exp(-np.abs(s0 - s1)))
    return np.allclose(o, o_ref, atol=1e-14) and np.allclose(lse, lse_ref, atol=1e-14)


def _pin_key_shift(fn):
    """Adding u to every key shifts row i's scores by scale*q_i.u: O is
    unchanged and lse moves by exactly that amount (softmax is per query row)."""
    rng = np.random.default_rng(16)
    q, k, v = _rand(rng, 5, 4), _rand(rng, 7, 4), _rand(rng, 7, 3)
    u = 4.0 * _rand(rng, 4)
    o1, l1 = fn(q, k, v, 0.6, False)
    o2, l2 = fn(q, k + u[None], v, 0.6, False)
    return np.allclose(o1, o2, atol=1e-12) and np.allclose(l2 - l1, 0.6 * (q @ u), atol=1e-12)


def _pin_permutation(fn):
    rng = np.random.default_rng(17)
    q, k, v = _rand(rng, 5, 4), _rand(rng, 9, 4), _rand(rng, 9, 3)
    perm = rng.permutation(9)
    o1, l1 = fn(q, k, v, 0.4, False)
    o2, l2 = fn(q, k[perm], v[perm], 0.4, False)
    return np.allclose(o1, o2, atol=1e-14) and np.allclose(l1, l2, atol=1e-14)


def _pin_brute(fn):
    rng = np.random.default_rng(18)
    ok = True
    for tq, tkv, causal in [(5, 5, False), (5, 5, True), (3, 7, True), (4, 6, False), (1, 6, True)]:
        q, k, v = _rand(rng, tq, 3), 2 * _rand(rng, tkv, 3), _rand(rng, tkv, 2)
        o, lse = fn(q, k, v, 0.8, causal)
        ob, lb = _brute(q, k, v, 0.8, causal)
        ok = ok and np.allclose(o, ob, rtol=1e-13, atol=1e-14) and np.allclose(lse, lb, rtol=1e-13, atol=1e-14)
    return ok


def _pin_torch_sdpa(fn):
    """Library cross-check: PyTorch's CPU attention in float64 (top-left
    causal alignment, which equals ours when T_q == T_kv)."""
    rng = np.random.default_rng(19)
    ok = True
    for causal in (False, True):
        q, k, v = _rand(rng, 16, 8), _rand(rng, 16, 8), _rand(rng, 16, 8)
        o, _ = fn(q, k, v, 0.3, causal)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
            torch.from_numpy(v)[None, None], is_causal=causal, scale=0.3)[0, 0].numpy()
        ok = ok and np.allclose(o, ref, rtol=1e-12, atol=1e-13)
    return ok


def _pin_causal_suffix(fn):
    """Bottom-right causal: the last T_q rows of a T x T causal problem are the
    T_q-query causal problem over the same keys (one new query sees every
    cached key), and T_q = 1 causal is plain attention over all keys."""
    rng = np.random.default_rng(20)
    qf, k, v = _rand(rng, 9, 4), _rand(rng, 9, 4), _rand(rng, 9, 3)
    of, lf = fn(qf, k, v, 0.5, True)
    o3, l3 = fn(qf[-3:], k, v, 0.5, True)
    o1, l1 = fn(qf[-1:], k, v, 0.5, True)
    on, ln_ = fn(qf[-1:], k, v, 0.5, False)
    return (np.allclose(o3, of[-3:], atol=1e-14) and np.allclose(l3, lf[-3:], atol=1e-14)
            and np.allclose(o1, on, atol=1e-15) and np.allclose(l1, ln_, atol=1e-15))


PIN_CHECKS = {
    "tkv1": _pin_tkv1,
    "zero_query": _pin_zero_query,
    "ones_value": _pin_ones_value,
    "causal_row0": _pin_causal_row0,
    "two_keys": _pin_two_keys,
    "key_shift": _pin_key_shift,
    "permutation": _pin_permutation,
    "brute_force": _pin_brute,
    "torch_sdpa": _pin_torch_sdpa,
    "causal_suffix": _pin_causal_suffix,
}


def _oracle_2d(q, k, v, scale, causal):
    return attention(q, k, v, scale, causal)


@pytest.mark.parametrize("name", sorted(PIN_CHECKS))
def test_oracle_pin(name):
    assert PIN_CHECKS[name](_oracle_2d)


# Plausible mistakes, planted in copies of the oracle (CPU only).  Each must
# be rejected by at least one pin.

def _mut_no_scale(q, k, v, scale, causal):
    return attention(q, k, v, 1.0, causal)


def _mut_wrong_axis(q, k, v, scale, causal):
    s = (q @ k.T) * scale
    if causal:
        tq, tkv = s.shape
        s[np.arange(tkv)[None, :] > np.arange(tq)[:, None] + tkv - tq] = -np.inf
    m = s.max(axis=0, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=0, keepdims=True)
    p = p / l
    return p @ v, (m + np.log(l)).ravel()[: s.shape[0]] if s.shape[1] >= s.shape[0] else np.zeros(s.shape[0])


def _mut_flipped_mask(q, k, v, scale, causal):
    if not causal:
        return attention(q, k, v, scale, False)
    s = (q @ k.T) * scale
    tq, tkv = s.shape
    s[np.arange(tkv)[None, :] < np.arange(tq)[:, None] + tkv - tq] = -np.inf
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    return (p @ v) / l[:, None], m + np.log(l)


def _mut_strict_diagonal(q, k, v, scale, causal):
    if not causal:
        return attention(q, k, v, scale, False)
    s = (q @ k.T) * scale
    tq, tkv = s.shape
    s[np.arange(tkv)[None, :] >= np.arange(tq)[:, None] + tkv - tq] = -np.inf
    s[0, 0] = 0.0 if tq == tkv else s[0, 0]
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    return (p @ v) / l[:, None], m + np.log(l)


def _mut_top_left_causal(q, k, v, scale, causal):
    if not causal:
        return attention(q, k, v, scale, False)
    s = (q @ k.T) * scale
    tq, tkv = s.shape
    s[np.arange(tkv)[None, :] > np.arange(tq)[:, None]] = -np.inf
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    return (p @ v) / l[:, None], m + np.log(l)


def _mut_lse_drops_max(q, k, v, scale, causal):
    o, lse = attention(q, k, v, scale, causal)
    s = (q @ k.T) * scale
    if causal:
        tq, tkv = s.shape
        s[np.arange(tkv)[None, :] > np.arange(tq)[:, None] + tkv - tq] = -np.inf
    return o, lse - s.max(axis=1)


def _mut_log2_lse(q, k, v, scale, causal):
    o, lse = attention(q, k, v, scale, causal)
    return o, lse / math.log(2.0)


def _mut_no_normalise(q, k, v, scale, causal):
    s = (q @ k.T) * scale
    if causal:
        tq, tkv = s.shape
        s[np.arange(tkv)[None, :] > np.arange(tq)[:, None] + tkv - tq] = -np.inf
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return p @ v, m + np.log(p.sum(axis=1))


def _mut_transposed_value(q, k, v, scale, causal):
    o, lse = attention(q, k, v, scale, causal)
    vv = v[::-1].copy()
    o2, _ = attention(q, k, vv, scale, causal)
    return o2, lse


def _mut_key_query_swapped(q, k, v, scale, causal):
    # uses k as queries against q as keys when shapes allow it
    if q.shape == k.shape:
        s = (k @ q.T) * scale
    else:
        s = (q @ k.T) * scale
    if causal:
        tq, tkv = s.shape
        s[np.arange(tkv)[None, :] > np.arange(tq)[:, None] + tkv - tq] = -np.inf
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    return (p @ v) / l[:, None], m + np.log(l)


MUTANTS = {
    "no_scale": _mut_no_scale,
    "wrong_axis": _mut_wrong_axis,
    "flipped_mask": _mut_flipped_mask,
    "strict_diagonal": _mut_strict_diagonal,
    "top_left_causal": _mut_top_left_causal,
    "lse_drops_max": _mut_lse_drops_max,
    "log2_lse": _mut_log2_lse,
    "no_normalise": _mut_no_normalise,
    "reversed_value_rows": _mut_transposed_value,
    "key_query_swapped": _mut_key_query_swapped,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name):
    fn = MUTANTS[name]
    failed = []
    for pin, check in PIN_CHECKS.items():
        try:
            ok = check(fn)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin)
    assert failed, f"mutant {name} passed every pin"


# ---------------------------------------------------------------- API behaviour

def test_rows_argument_matches_full_rows():
    rng = np.random.default_rng(21)
    q, k, v = _rand(rng, 2, 3, 12, 4), _rand(rng, 2, 3, 12, 4), _rand(rng, 2, 3, 12, 5)
    rows = np.array([0, 5, 11, 3])
    for causal in (False, True):
        o, lse = attention(q, k, v, 0.5, causal)
        o_r, lse_r = attention(q, k, v, 0.5, causal, rows=rows)
        np.testing.assert_array_equal(o_r, o[..., rows, :])
        np.testing.assert_array_equal(lse_r, lse[..., rows])


def test_leading_axes_are_independent():
    rng = np.random.default_rng(22)
    q, k, v = _rand(rng, 2, 3, 6, 4), _rand(rng, 2, 3, 8, 4), _rand(rng, 2, 3, 8, 5)
    o, lse = attention(q, k, v, 0.5, True)
    for b in range(2):
        for h in range(3):
            ob, lb = attention(q[b, h], k[b, h], v[b, h], 0.5, True)
            np.testing.assert_array_equal(o[b, h], ob)
            np.testing.assert_array_equal(lse[b, h], lb)


def test_causal_query_longer_than_keys_rejected():
    rng = np.random.default_rng(23)
    with pytest.raises(ValueError):
        attention(_rand(rng, 5, 4), _rand(rng, 4, 4), _rand(rng, 4, 2), 0.5, causal=True)


def test_large_scores_are_stable():
    rng = np.random.default_rng(24)
    q, k, v = 40.0 * _rand(rng, 4, 8), 40.0 * _rand(rng, 16, 8), _rand(rng, 16, 3)
    o, lse = attention(q, k, v, 1.0, False)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    ob, lb = _brute(q, k, v, 1.0, False)
    np.testing.assert_allclose(o, ob, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, lb, rtol=1e-13)


@pytest.mark.parametrize("num_splits", [1, 2, 3, 16, 40, 43])
def test_split_combine_equals_unsplit(num_splits):
    rng = np.random.default_rng(25)
    q, k, v = _rand(rng, 2, 3, 1, 8), 3 * _rand(rng, 2, 3, 40, 8), _rand(rng, 2, 3, 40, 6)
    o, lse = attention(q, k, v, 0.35)
    o_s, lse_s = oracle.split_attention(q, k, v, 0.35, num_splits)
    np.testing.assert_allclose(o_s, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse_s, lse, rtol=1e-13, atol=1e-13)


def test_combine_closed_forms():
    # two partitions with equal normalisers: the plain mean, and lse + ln 2
    o1, o2 = np.array([[1.0, -2.0]]), np.array([[3.0, 4.0]])
    lse = np.array([0.7])
    o, l = oracle.combine_partials(np.stack([o1, o2]), np.stack([lse, lse]))
    np.testing.assert_allclose(o, (o1 + o2) / 2, rtol=1e-15)
    np.testing.assert_allclose(l, lse + math.log(2.0), rtol=1e-15)
    # a partition with no keys (lse = -inf) has zero weight, whatever its
    # (finite) output
    o3 = np.array([[1e30, -7.0]])
    o, l = oracle.combine_partials(np.stack([o1, o3]), np.stack([lse, np.array([-np.inf])]))
    np.testing.assert_array_equal(o, o1)
    np.testing.assert_array_equal(l, lse)
    # weights follow exp(lse_p): a partition e^5 times heavier dominates by that factor
    o, l = oracle.combine_partials(np.stack([o1, o2]), np.stack([lse, lse + 5.0]))
    w = math.exp(5.0)
    np.testing.assert_allclose(o, (o1 + w * o2) / (1 + w), rtol=1e-14)
    np.testing.assert_allclose(l, lse + math.log1p(w), rtol=1e-14)


def test_combine_is_order_free():
    rng = np.random.default_rng(27)
    o_p, lse_p = rng.standard_normal((5, 3, 4)), 4 * rng.standard_normal((5, 3))
    o, l = oracle.combine_partials(o_p, lse_p)
    perm = rng.permutation(5)
    o2, l2 = oracle.combine_partials(o_p[perm], lse_p[perm])
    np.testing.assert_allclose(o2, o, rtol=1e-13)
    np.testing.assert_allclose(l2, l, rtol=1e-14)


def test_split_below_one_raises():
    rng = np.random.default_rng(26)
    with pytest.raises(ValueError):
        oracle.split_attention(_rand(rng, 1, 4), _rand(rng, 4, 4), _rand(rng, 4, 2), 0.5, 0)


# ---------------------------------------------------------------- grouped-query heads

def test_gqa_with_one_query_head_per_group_is_attention():
    rng = np.random.default_rng(30)
    q, k, v = _rand(rng, 2, 4, 3, 8), _rand(rng, 2, 4, 9, 8), _rand(rng, 2, 4, 9, 5)
    for causal in (False, True):
        o1, l1 = oracle.attention_gqa(q, k, v, 0.4, causal)
        o2, l2 = attention(q, k, v, 0.4, causal)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_gqa_equals_attention_on_repeated_heads():
    """H_kv heads each shared by G query heads == full attention with every
    key/value head repeated G times (consecutive query heads share one)."""
    rng = np.random.default_rng(31)
    B, hkv, G = 2, 3, 4
    q = _rand(rng, B, hkv * G, 2, 8)
    k, v = _rand(rng, B, hkv, 11, 8), _rand(rng, B, hkv, 11, 6)
    o, lse = oracle.attention_gqa(q, k, v, 0.3)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    ob, lb = _brute(q[1, 7], kr[1, 7], vr[1, 7], 0.3, False)
    np.testing.assert_allclose(o[1, 7], ob, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse[1, 7], lb, rtol=1e-13)
    o2, l2 = attention(q, kr, vr, 0.3)
    np.testing.assert_allclose(o, o2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse, l2, rtol=1e-14)
    # query head 5 belongs to group 1 (heads 4..7): it must ignore kv heads 0 and 2
    k_alt = k.copy()
    k_alt[:, 0] += 5.0
    k_alt[:, 2] -= 5.0
    o3, _ = oracle.attention_gqa(q, k_alt, v, 0.3)
    np.testing.assert_array_equal(o3[:, 5], o[:, 5])


def test_gqa_rejects_uneven_groups():
    rng = np.random.default_rng(32)
    with pytest.raises(ValueError):
        oracle.attention_gqa(_rand(rng, 1, 6, 1, 4), _rand(rng, 1, 4, 5, 4), _rand(rng, 1, 4, 5, 4), 0.5)


def test_combine_is_shift_invariant():
    """Adding c to every partition's log-sum-exp scales every weight by e^c:
    the merged output is unchanged and the merged LSE moves by c, also where
    e^lse itself is past the float64 range (scores of a few hundred)."""
    rng = np.random.default_rng(28)
    o_p, lse_p = rng.standard_normal((4, 3, 5)), rng.standard_normal((4, 3))
    o, l = oracle.combine_partials(o_p, lse_p)
    eps = np.finfo(np.float64).eps
    for c in (-900.0, 750.0, 1e4):
        o2, l2 = oracle.combine_partials(o_p, lse_p + c)
        assert np.isfinite(o2).all() and np.isfinite(l2).all(), c
        # lse_p + c rounds at |c| eps / 2 absolute, so each weight carries a
        # relative error up to about |c| eps (two such roundings per ratio)
        tol = 4 * abs(c) * eps * np.abs(o_p).max() + 1e-14
        np.testing.assert_allclose(o2, o, rtol=0, atol=tol)
        np.testing.assert_allclose(l2, l + c, rtol=0, atol=4 * abs(c) * eps + 1e-14)


# ------------------------------------------- planted mistakes beyond attention()
#
# Copies of the recurrence, the one-query online form, the partition merge, the
# split and the grouped-query mapping, each with one plausible mistake.  Each is
# installed in place of the original (in the package and in its defining
# module, so internal callers see it too) and must fail at least one of the
# pins above.

_ATT = __import__("sys").modules["oracle.attention"]


def _states_with_merge(merge):
    """online_softmax_states with its merge step replaced."""
    def states(scores, block):
        if block < 1:
            raise ValueError("block must be at least 1")
        s = np.asarray(scores, dtype=np.float64).ravel()
        run, out = (-math.inf, 0.0), []
        for i in range(0, s.size, block):
            sb = s[i:i + block]
            m_b = float(sb.max())
            run = merge(run, (m_b, float(np.exp(sb - m_b).sum())))
            out.append(run)
        return out
    return states


def _merge_no_rescale(run, blk):
    m_new = max(run[0], blk[0])
    return m_new, run[1] + blk[1] * math.exp(blk[0] - m_new)       # old sum not rescaled


def _merge_inverted_rescale(run, blk):
    m_new = max(run[0], blk[0])
    w = math.exp(m_new - run[0]) if run[1] else 0.0                 # exponent upside down
    return m_new, w * run[1] + blk[1] * math.exp(blk[0] - m_new)


def _merge_block_max_only(run, blk):
    m_new = blk[0]                                                  # running max forgotten
    w = math.exp(run[0] - m_new) if run[1] else 0.0
    return m_new, w * run[1] + blk[1]


_mut_states_no_rescale = _states_with_merge(_merge_no_rescale)
_mut_states_inverted_rescale = _states_with_merge(_merge_inverted_rescale)
_mut_states_block_max_only = _states_with_merge(_merge_block_max_only)


def _online_variant(rescale_acc=True, rescale_sum=True, scaled=True):
    def online(q, K, V, block):
        if block < 1:
            raise ValueError("block must be at least 1")
        q, K, V = (np.asarray(x, dtype=np.float64) for x in (q, K, V))
        scale = 1.0 / math.sqrt(q.shape[0]) if scaled else 1.0
        m, l, acc = -math.inf, 0.0, np.zeros(V.shape[1])
        for i in range(0, K.shape[0], block):
            sb = (K[i:i + block] @ q) * scale
            m_b = float(sb.max())
            e = np.exp(sb - m_b)
            m_new = max(m, m_b)
            w_run = 0.0 if m == -math.inf else math.exp(m - m_new)
            w_blk = math.exp(m_b - m_new)
            l = (w_run * l if rescale_sum else l) + w_blk * float(e.sum())
            acc = (w_run * acc if rescale_acc else acc) + w_blk * (e @ V[i:i + block])
            m = m_new
        return acc / l
    return online


def _mut_combine_mean(o_parts, lse_parts):
    o_parts, lse_parts = np.asarray(o_parts, np.float64), np.asarray(lse_parts, np.float64)
    M = lse_parts.max(axis=0)
    return o_parts.mean(axis=0), M + np.log(np.exp(lse_parts - M[None]).sum(axis=0))


def _mut_combine_lse_is_max(o_parts, lse_parts):
    o, _ = oracle.attention_module_combine(o_parts, lse_parts)
    return o, np.asarray(lse_parts, np.float64).max(axis=0)


def _mut_combine_unshifted(o_parts, lse_parts):
    o_parts, lse_parts = np.asarray(o_parts, np.float64), np.asarray(lse_parts, np.float64)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        w = np.exp(lse_parts)                            # no max subtracted
        wsum = w.sum(axis=0)
        return (w[..., None] * o_parts).sum(axis=0) / wsum[..., None], np.log(wsum)


def _mut_combine_divides_by_count(o_parts, lse_parts):
    o_parts, lse_parts = np.asarray(o_parts, np.float64), np.asarray(lse_parts, np.float64)
    M = lse_parts.max(axis=0)
    w = np.exp(lse_parts - M[None])
    return (w[..., None] * o_parts).sum(axis=0) / lse_parts.shape[0], M + np.log(w.sum(axis=0))


def _split_variant(shift_hi=0, shift_lo=0):
    def split(q, k, v, scale, num_splits):
        if num_splits < 1:
            raise ValueError("num_splits must be at least 1")
        k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
        tkv = k.shape[-2]
        o_parts, lse_parts = [], []
        for p in range(num_splits):
            lo = max(0, (p * tkv) // num_splits + (shift_lo if p else 0))
            hi = ((p + 1) * tkv) // num_splits + (shift_hi if p < num_splits - 1 else 0)
            if hi <= lo:
                continue
            o_p, lse_p = attention(q, k[..., lo:hi, :], v[..., lo:hi, :], scale)
            o_parts.append(o_p)
            lse_parts.append(lse_p)
        return _ATT.combine_partials(np.stack(o_parts), np.stack(lse_parts))
    return split


def _mut_gqa_modulo(q, k, v, scale, causal=False, rows=None):
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    hq, hkv = q.shape[1], k.shape[1]
    if hq % hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    outs = [attention(q[:, h], k[:, h % hkv], v[:, h % hkv], scale, causal, rows) for h in range(hq)]
    return np.stack([o for o, _ in outs], axis=1), np.stack([l for _, l in outs], axis=1)


_RECURRENCE_PINS = [
    test_worked_example_after_block_1,
    test_worked_example_final_state_equals_full_row,
    test_worked_example_split_into_its_two_blocks,
    lambda: test_blockwise_equals_full_for_every_block_size(7),
    lambda: test_blockwise_equals_full_for_every_block_size(17),
]
_COMBINE_PINS = [
    test_worked_example_split_into_its_two_blocks,
    test_combine_closed_forms,
    test_combine_is_order_free,
    test_combine_is_shift_invariant,
    lambda: test_split_combine_equals_unsplit(3),
    lambda: test_split_combine_equals_unsplit(16),
]
_GQA_PINS = [test_gqa_with_one_query_head_per_group_is_attention, test_gqa_equals_attention_on_repeated_heads]

MORE_MUTANTS = {  # name -> (function replaced, mutant, pins that must catch it)
    "states_no_rescale": ("online_softmax_states", _mut_states_no_rescale, _RECURRENCE_PINS),
    "states_inverted_rescale": ("online_softmax_states", _mut_states_inverted_rescale, _RECURRENCE_PINS),
    "states_block_max_only": ("online_softmax_states", _mut_states_block_max_only, _RECURRENCE_PINS),
    "online_acc_not_rescaled": ("online_attention", _online_variant(rescale_acc=False), _RECURRENCE_PINS),
    "online_sum_not_rescaled": ("online_attention", _online_variant(rescale_sum=False), _RECURRENCE_PINS),
    "online_unscaled_scores": ("online_attention", _online_variant(scaled=False), _RECURRENCE_PINS),
    "combine_plain_mean": ("combine_partials", _mut_combine_mean, _COMBINE_PINS),
    "combine_lse_is_max": ("combine_partials", _mut_combine_lse_is_max, _COMBINE_PINS),
    "combine_unshifted_weights": ("combine_partials", _mut_combine_unshifted, _COMBINE_PINS),
    "combine_divides_by_count": ("combine_partials", _mut_combine_divides_by_count, _COMBINE_PINS),
    "split_drops_last_key": ("split_attention", _split_variant(shift_hi=-1), _COMBINE_PINS),
    "split_overlapping_partitions": ("split_attention", _split_variant(shift_lo=-1), _COMBINE_PINS),
    "gqa_modulo_heads": ("attention_gqa", _mut_gqa_modulo, _GQA_PINS),
}


@pytest.mark.parametrize("name", sorted(MORE_MUTANTS))
def test_pins_reject_planted_mistake_beyond_attention(name, monkeypatch):
    target, mutant, pins = MORE_MUTANTS[name]
    # the combine mutant that keeps the original output needs the original
    monkeypatch.setattr(oracle, "attention_module_combine", _ATT.combine_partials, raising=False)
    monkeypatch.setattr(oracle, target, mutant)
    monkeypatch.setattr(_ATT, target, mutant)
    caught = 0
    for pin in pins:
        try:
            pin()
        except Exception:          # an assertion, or a failure inside the mutant
            caught += 1
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_pins_pass():
    """The same pin lists, run on the oracle as it is, all pass (so that a
    mutant counts as caught only by its mistake)."""
    for pin in _RECURRENCE_PINS + _COMBINE_PINS + _GQA_PINS:
        pin()
