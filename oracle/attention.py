"""Float64 CPU oracle for the exact attention forward -- test infrastructure.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this module.  It is deliberately the plain definition: the
score matrix S and the probabilities P are materialised for a whole head, with
no blocking, fusion or reordering beyond what the pages state.

Conventions (the pages leave these open; the readings taken are listed in the
design notes):

* Layout: q is (..., T_q, d), k and v are (..., T_kv, d); all leading axes are
  independent (batch, head) slices.
* ``scale`` multiplies q.k; the pages use 1/sqrt(d).
* Causal: key j is visible to query i iff j <= i + (T_kv - T_q).  For
  self-attention (T_q == T_kv) this is "position i sees the keys up to and
  including itself", which gives the T(T+1)/2 pair count of "Attention and
  Its Computational Cost", section "What is being computed".  Causal with
  T_q > T_kv would leave rows with no keys and is rejected.
* LSE is the natural-log normaliser of each row in units of the scaled score:
  lse_i = m_i + ln(l_i) = ln sum_j exp(scale * q_i . k_j).
"""

from __future__ import annotations

import math

import numpy as np


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def attention(q, k, v, scale: float, causal: bool = False, rows=None):
    """The definition, materialised.

    "FlashAttention IO-aware tiling lab", kernel-phase captions: S = QK^T /
    sqrt(d), P = softmax(S), O = PV.  "Attention and Its Computational Cost",
    "What is being computed": S and P are both T_q x T_kv; causal
    self-attention keeps T(T+1)/2 of the pairs.

    Steps, per leading slice:
      1. S = (Q K^T) * scale                         (T_q x T_kv)
      2. causal: S[i, j] = -inf where j > i + T_kv - T_q
      3. m_i = max_j S[i, j];  P = exp(S - m);  l_i = sum_j P[i, j]
      4. O = (P V) / l;  lse_i = m_i + ln l_i

    ``rows`` (optional, 1-D int array) restricts the computation to those query
    rows of the full T_q-row problem; the causal mask still uses each row's
    absolute index, so the result equals the same rows of the full answer.

    Returns (o, lse) as float64 arrays of shape (..., R, d_v) and (..., R),
    where R is T_q or len(rows).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    if q.ndim < 2 or k.ndim != q.ndim or v.ndim != q.ndim:
        raise ValueError("q, k, v must have the same rank >= 2")
    tq, d = q.shape[-2], q.shape[-1]
    tkv = k.shape[-2]
    if k.shape[-1] != d or v.shape[-2] != tkv or k.shape[:-2] != q.shape[:-2] or v.shape[:-2] != q.shape[:-2]:
        raise ValueError("shape mismatch between q, k, v")
    if tq < 1 or tkv < 1 or d < 1:
        raise ValueError("sizes must be >= 1")
    if causal and tq > tkv:
        raise ValueError("causal attention needs T_q <= T_kv (every row must see a key)")
    row_idx = np.arange(tq) if rows is None else np.asarray(rows, dtype=np.int64)
    lead = q.shape[:-2]
    dv = v.shape[-1]
    qf = q.reshape((-1, tq, d))
    kf = k.reshape((-1, tkv, d))
    vf = v.reshape((-1, tkv, dv))
    n = qf.shape[0]
    o_out = np.empty((n, row_idx.size, dv))
    lse_out = np.empty((n, row_idx.size))
    if causal:
        # visible[i, j] is True iff key j may be seen by query row_idx[i]
        visible = np.arange(tkv)[None, :] <= (row_idx[:, None] + (tkv - tq))
    for s in range(n):
        scores = qf[s, row_idx] @ kf[s].T          # step 1 (unscaled product)
        scores *= scale
        if causal:                                  # step 2
            scores[~visible] = -np.inf
        m = scores.max(axis=1)                      # step 3
        np.subtract(scores, m[:, None], out=scores)
        np.exp(scores, out=scores)                  # scores now holds P
        l = scores.sum(axis=1)
        o_out[s] = (scores @ vf[s]) / l[:, None]    # step 4
        lse_out[s] = m + np.log(l)
    return o_out.reshape(lead + (row_idx.size, dv)), lse_out.reshape(lead + (row_idx.size,))


def attention_gqa(q, k, v, scale: float, causal: bool = False, rows=None):
    """Grouped-query attention: q is (B, H_q, T_q, d), k and v are
    (B, H_kv, T_kv, d) with H_q a multiple of H_kv; query head h attends key /
    value head h // (H_q / H_kv).

    "Attention and Its Computational Cost", "The other shape: one query, many
    keys": grouped-query attention keeps fewer key and value heads than query
    heads, cutting the cache that every decode step reads.  Each query head is
    the plain definition (``attention``) against its group's key/value head.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be (B, H, T, d)")
    B, hq = q.shape[0], q.shape[1]
    hkv = k.shape[1]
    if hkv < 1 or hq % hkv != 0 or v.shape[1] != hkv or k.shape[0] != B or v.shape[0] != B:
        raise ValueError("H_q must be a multiple of H_kv")
    group = hq // hkv
    outs, lses = [], []
    for h in range(hq):
        o_h, l_h = attention(q[:, h], k[:, h // group], v[:, h // group], scale, causal, rows)
        outs.append(o_h)
        lses.append(l_h)
    return np.stack(outs, axis=1), np.stack(lses, axis=1)


def standard_attention(q, K, V):
    """One query against a full key set, score vector materialised.

    "E8.1 IO-aware attention", "Do it in code": softmax(K q / sqrt(d)) V for a
    single query.  Returns the d_v-vector output.
    """
    q = _as_f64(q)
    K = _as_f64(K)
    V = _as_f64(V)
    s = (K @ q) / math.sqrt(q.shape[0])
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def _block_summary(s, vb=None):
    """One block's own softmax state, relative to its own maximum m_b: the
    sum of exp(s_j - m_b) and (when values are given) the exp-weighted sum
    of its value rows."""
    m_b = float(s.max())
    e = np.exp(s - m_b)
    return m_b, float(e.sum()), (None if vb is None else e @ vb)


def _rescale_merge(run, blk):
    """The running state (m, l, acc) extended by a block's summary: both are
    put on the common reference max(m, m_b), each side multiplied by
    exp(its own reference - the common one).  An empty running state
    (m = -inf) gets weight 0."""
    m, l, acc = run
    m_b, l_b, acc_b = blk
    m_new = max(m, m_b)
    w_run = 0.0 if m == -math.inf else math.exp(m - m_new)
    w_blk = math.exp(m_b - m_new)
    acc_new = None if acc_b is None else w_run * acc + w_blk * acc_b
    return m_new, w_run * l + w_blk * l_b, acc_new


def online_softmax_states(scores, block: int):
    """Running (m, l) after each block of a score row.

    "IO-Aware Attention: Tiling the Score Matrix Without Materializing It",
    section "Softmax over blocks, exactly": after each block the running
    maximum is the larger of the previous one and the block's, and the
    running sum is re-expressed relative to it, the part accumulated so far
    scaled by exp(old max - new max).  Start: m = -inf, l = 0.  Here each
    block is first summarised on its own maximum and then merged into the
    running state (``_rescale_merge``), which gives the same (m, l).

    Returns a list of (m, l) pairs, one per block, in block order.
    """
    if block < 1:
        raise ValueError("block must be at least 1")
    s = _as_f64(scores).ravel()
    state = (-math.inf, 0.0, None)
    states = []
    for start in range(0, s.size, block):
        state = _rescale_merge(state, _block_summary(s[start:start + block]))
        states.append((state[0], state[1]))
    return states


def online_attention(q, K, V, block: int):
    """The blockwise online form for one query, never holding more than one
    block of scores.

    "E8.1 IO-aware attention", "Do it in code": a function of one query, the
    keys, the values and the block size (below 1 it raises ValueError) that
    walks the keys block by block.  Each block's scores (scale 1/sqrt(d)) are
    summarised on their own maximum, merged into the running (m, l, weighted
    value sum) with the rescaling of "IO-Aware Attention", section "Softmax
    over blocks, exactly", and the weighted sum is divided by l once, after
    the last block.
    """
    if block < 1:
        raise ValueError("block must be at least 1")
    q = _as_f64(q)
    K = _as_f64(K)
    V = _as_f64(V)
    scale = 1.0 / math.sqrt(q.shape[0])
    state = (-math.inf, 0.0, np.zeros(V.shape[1]))
    for start in range(0, K.shape[0], block):
        scores = (K[start:start + block] @ q) * scale
        state = _rescale_merge(state, _block_summary(scores, V[start:start + block]))
    _, l, acc = state
    return acc / l


def combine_partials(o_parts, lse_parts):
    """Merge per-partition results with the softmax rescaling.

    "IO-Aware Attention: Tiling the Score Matrix Without Materializing It",
    section "Parallelism and the cost of the split": each key partition yields
    a partial output and a partial normaliser, merged with the same rescaling
    recurrence applied across partitions.  With partition p holding the
    normalised output O_p and lse_p = ln(l_p) + m_p:
        M = max_p lse_p,  w_p = exp(lse_p - M),
        lse = M + ln(sum_p w_p),  O = sum_p w_p O_p / sum_p w_p.

    o_parts: (P, ..., d_v), lse_parts: (P, ...).  Partitions with lse = -inf
    (no keys) get zero weight; their outputs must be finite (0 * nan is nan).
    At least one partition of each row must have keys.
    """
    o_parts = _as_f64(o_parts)
    lse_parts = _as_f64(lse_parts)
    M = lse_parts.max(axis=0)
    w = np.exp(lse_parts - M[None])
    wsum = w.sum(axis=0)
    o = (w[..., None] * o_parts).sum(axis=0) / wsum[..., None]
    return o, M + np.log(wsum)


def split_attention(q, k, v, scale: float, num_splits: int):
    """Non-causal attention over key partitions, then merged.

    Partition p covers keys [floor(p T / P), floor((p + 1) T / P)); each one
    is the plain definition (``attention``) on its keys, and the partials are
    merged by ``combine_partials``.  Empty partitions (P > T) are skipped.
    """
    if num_splits < 1:
        raise ValueError("num_splits must be at least 1")
    k = _as_f64(k)
    v = _as_f64(v)
    tkv = k.shape[-2]
    o_parts, lse_parts = [], []
    for p in range(num_splits):
        lo = (p * tkv) // num_splits
        hi = ((p + 1) * tkv) // num_splits
        if hi <= lo:
            continue
        o_p, lse_p = attention(q, k[..., lo:hi, :], v[..., lo:hi, :], scale)
        o_parts.append(o_p)
        lse_parts.append(lse_p)
    return combine_partials(np.stack(o_parts), np.stack(lse_parts))
