"""Float64 CPU oracle for the attention backward pass -- test infrastructure.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this module.  For an upstream gradient dO of the output O of
the forward definition (``oracle.attention``), the gradients are those of the
plain definition, written out per (batch, head) slice with S and P
materialised:

    S = scale * Q K^T (masked entries -inf),  P = softmax_rows(S),  O = P V
    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij            (= sum_d dO_id O_id)
    dS = P * (dP - D)                 (elementwise; zero where masked)
    dQ = scale * dS K,   dK = scale * dS^T Q

"IO-Aware Attention: Tiling the Score Matrix Without Materializing It",
section "What has to stay in fast memory": the forward keeps only O and one
normaliser per query row, so the probabilities the gradients use are rebuilt
from Q, K, V and those per-row values.  ``attention_backward_from_lse`` follows that
route (P = exp(S - lse), D from dO and O); ``attention_backward`` is the plain
definition.  The derivative formulas themselves are not on the pages; they
are the calculus of the forward definition and are pinned in
``tests/test_oracle_backward.py`` by central finite differences of the
forward oracle, by PyTorch float64 autograd, and by identities.
"""

from __future__ import annotations

import numpy as np


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _slices(q, k, v, do):
    q, k, v, do = (_as_f64(t) for t in (q, k, v, do))
    if q.ndim < 2 or not (q.ndim == k.ndim == v.ndim == do.ndim):
        raise ValueError("q, k, v, dO must have the same rank >= 2")
    tq, d = q.shape[-2:]
    tkv = k.shape[-2]
    if k.shape[-1] != d or v.shape[-2] != tkv or do.shape[-2:] != (tq, v.shape[-1]):
        raise ValueError("shape mismatch between q, k, v, dO")
    lead = q.shape[:-2]
    return (q.reshape(-1, tq, d), k.reshape(-1, tkv, d), v.reshape(-1, tkv, v.shape[-1]),
            do.reshape(-1, tq, v.shape[-1]), lead, tq, tkv)


def _visible(tq: int, tkv: int, causal: bool):
    if not causal:
        return None
    if tq > tkv:
        raise ValueError("causal attention needs T_q <= T_kv (every row must see a key)")
    # key j visible to query i iff j <= i + (T_kv - T_q)  (bottom-right alignment)
    return np.arange(tkv)[None, :] <= (np.arange(tq)[:, None] + (tkv - tq))


def _grads(p, qs, ks, vs, dos, D, scale):
    dv = p.T @ dos
    dp = dos @ vs.T
    ds = p * (dp - D[:, None])
    return scale * (ds @ ks), scale * (ds.T @ qs), dv


def attention_backward(q, k, v, do, scale: float, causal: bool = False):
    """Gradients (dq, dk, dv) of sum(O * dO) for O = attention(q, k, v), plus
    D (the per-row constant sum_j P_ij dP_ij), all float64."""
    qf, kf, vf, dof, lead, tq, tkv = _slices(q, k, v, do)
    vis = _visible(tq, tkv, causal)
    dq, dk, dv = np.empty_like(qf), np.empty_like(kf), np.empty_like(vf)
    Dout = np.empty((qf.shape[0], tq))
    for s in range(qf.shape[0]):
        sc = (qf[s] @ kf[s].T) * scale
        if vis is not None:
            sc[~vis] = -np.inf
        p = np.exp(sc - sc.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        D = (p * (dof[s] @ vf[s].T)).sum(axis=1)
        dq[s], dk[s], dv[s] = _grads(p, qf[s], kf[s], vf[s], dof[s], D, scale)
        Dout[s] = D
    return (dq.reshape(lead + dq.shape[1:]), dk.reshape(lead + dk.shape[1:]), dv.reshape(lead + dv.shape[1:]),
            Dout.reshape(lead + (tq,)))


def attention_backward_from_lse(q, k, v, o, do, lse, scale: float, causal: bool = False):
    """The recomputation route: P = exp(scale * Q K^T - lse) from the saved
    natural-log row constants, D_i = sum_d dO_id O_id from the saved output.
    Returns (dq, dk, dv, D)."""
    qf, kf, vf, dof, lead, tq, tkv = _slices(q, k, v, do)
    of = _as_f64(o).reshape(dof.shape)
    lf = _as_f64(lse).reshape(qf.shape[0], tq)
    vis = _visible(tq, tkv, causal)
    dq, dk, dv = np.empty_like(qf), np.empty_like(kf), np.empty_like(vf)
    Dout = np.empty((qf.shape[0], tq))
    for s in range(qf.shape[0]):
        sc = (qf[s] @ kf[s].T) * scale
        if vis is not None:
            sc[~vis] = -np.inf
        p = np.exp(sc - lf[s][:, None])
        D = (dof[s] * of[s]).sum(axis=1)
        dq[s], dk[s], dv[s] = _grads(p, qf[s], kf[s], vf[s], dof[s], D, scale)
        Dout[s] = D
    return (dq.reshape(lead + dq.shape[1:]), dk.reshape(lead + dk.shape[1:]), dv.reshape(lead + dv.shape[1:]),
            Dout.reshape(lead + (tq,)))
