"""Pins of the float64 backward oracle (oracle/backward.py) against what does
not share its arithmetic: central finite differences of the forward oracle,
PyTorch float64 autograd through its own attention routine, and identities of
the softmax Jacobian.  Planted mistakes must fail at least one pin."""

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as bw


def rand(rng, *shape):
    return rng.standard_normal(shape)


def loss_and_fd(q, k, v, do, scale, causal, h=1e-6):
    """Central differences of L = sum(O * dO) w.r.t. every element of q, k, v."""
    def loss(qq, kk, vv):
        o, _ = oracle.attention(qq, kk, vv, scale, causal)
        return float((o * do).sum())
    grads = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(base[which])
        it = np.nditer(g, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [t.copy() for t in base]
            minus = [t.copy() for t in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return grads


CASES = [  # B, H, Tq, Tkv, d, causal
    (1, 1, 3, 4, 2, False),
    (1, 2, 4, 4, 3, True),
    (2, 1, 2, 5, 2, True),    # bottom-right causal, Tq < Tkv
    (1, 1, 5, 1, 2, False),   # a single key
]


@pytest.mark.parametrize("B,H,Tq,Tkv,d,causal", CASES)
def test_matches_finite_differences(B, H, Tq, Tkv, d, causal):
    rng = np.random.default_rng(100 + Tq * 7 + Tkv)
    q, k, v, do = rand(rng, B, H, Tq, d), rand(rng, B, H, Tkv, d), rand(rng, B, H, Tkv, d), rand(rng, B, H, Tq, d)
    scale = 0.7
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, causal)
    fq, fk, fv = loss_and_fd(q, k, v, do, scale, causal)
    np.testing.assert_allclose(dq, fq, atol=1e-7)
    np.testing.assert_allclose(dk, fk, atol=1e-7)
    np.testing.assert_allclose(dv, fv, atol=1e-7)


@pytest.mark.parametrize("Tq,Tkv,causal", [(16, 16, False), (16, 16, True), (7, 20, True), (9, 13, False)])
def test_matches_torch_autograd(Tq, Tkv, causal):
    rng = np.random.default_rng(7 + Tq + Tkv)
    B, H, d, scale = 2, 3, 8, 1 / np.sqrt(8)
    q, k, v, do = rand(rng, B, H, Tq, d), rand(rng, B, H, Tkv, d), rand(rng, B, H, Tkv, d), rand(rng, B, H, Tq, d)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = None
    if causal:
        mask = torch.ones(Tq, Tkv, dtype=torch.bool).tril(diagonal=Tkv - Tq)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    o.backward(torch.tensor(do))
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, causal)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_identities(causal):
    rng = np.random.default_rng(3)
    B, H, T, d = 2, 2, 24, 5
    q, k, v, do = rand(rng, B, H, T, d), rand(rng, B, H, T, d), rand(rng, B, H, T, d), rand(rng, B, H, T, d)
    dq, dk, dv, D = oracle.attention_backward(q, k, v, do, 0.4, causal)
    # rows of dS sum to zero, so the key gradients sum to zero over the keys
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # rows of P sum to one, so the value gradients sum to the upstream gradients
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
    # D is the row sum of dO * O
    o, _ = oracle.attention(q, k, v, 0.4, causal)
    np.testing.assert_allclose(D, (do * o).sum(axis=-1), atol=1e-12)


def test_single_key_closed_form():
    rng = np.random.default_rng(4)
    q, k, v, do = rand(rng, 1, 1, 6, 3), rand(rng, 1, 1, 1, 3), rand(rng, 1, 1, 1, 3), rand(rng, 1, 1, 6, 3)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 1.0)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv[0, 0, 0], do[0, 0].sum(axis=0), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_recomputation_from_saved_row_constants(causal):
    rng = np.random.default_rng(5)
    B, H, Tq, Tkv, d = 1, 2, 20, 30, 4
    q, k, v, do = rand(rng, B, H, Tq, d), rand(rng, B, H, Tkv, d), rand(rng, B, H, Tkv, d), rand(rng, B, H, Tq, d)
    o, lse = oracle.attention(q, k, v, 0.5, causal)
    ref = oracle.attention_backward(q, k, v, do, 0.5, causal)
    got = oracle.attention_backward_from_lse(q, k, v, o, do, lse, 0.5, causal)
    for a, b in zip(ref, got):
        np.testing.assert_allclose(a, b, atol=1e-12)


def _mutant(kind):
    def grads(p, qs, ks, vs, dos, D, scale):
        dv = p.T @ dos
        dp = dos @ vs.T
        if kind == "no_D":
            ds = p * dp
        elif kind == "D_over_keys":
            ds = p * (dp - (p * dp).sum(axis=0)[None, :])
        else:
            ds = p * (dp - D[:, None])
        dq = scale * (ds @ ks)
        dk = scale * (ds.T @ qs)
        if kind == "dq_unscaled":
            dq = ds @ ks
        if kind == "dk_untransposed":
            dk = scale * (ds @ qs)
        if kind == "dv_untransposed":
            dv = p @ dos
        if kind == "dq_with_v":
            dq = scale * (ds @ vs)
        return dq, dk, dv
    return grads


@pytest.mark.parametrize("kind", ["no_D", "D_over_keys", "dq_unscaled", "dk_untransposed", "dv_untransposed",
                                  "dq_with_v"])
def test_planted_mistakes_fail_a_pin(kind, monkeypatch):
    rng = np.random.default_rng(6)
    B, H, T, d = 1, 1, 4, 4
    q, k, v, do = rand(rng, B, H, T, d), rand(rng, B, H, T, d), rand(rng, B, H, T, d), rand(rng, B, H, T, d)
    fq, fk, fv = loss_and_fd(q, k, v, do, 0.6, True)
    monkeypatch.setattr(bw, "_grads", _mutant(kind))
    dq, dk, dv, _ = bw.attention_backward(q, k, v, do, 0.6, True)
    err = max(np.abs(dq - fq).max(), np.abs(dk - fk).max(), np.abs(dv - fv).max())
    assert err > 1e-4, kind


def test_rejects_causal_with_more_queries_than_keys():
    z = np.zeros((1, 1, 3, 2))
    with pytest.raises(ValueError):
        oracle.attention_backward(z, z[:, :, :2], z[:, :, :2], z, 1.0, causal=True)
