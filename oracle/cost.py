"""Closed-form cost model for exact attention -- test infrastructure.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this module.  The functions restate the counting rules of:

* "Attention and Its Computational Cost" (programmer.ie), sections "What is
  being computed" (FLOPs), "The cost of writing down the scores" (score
  tensor size), "The other shape: one query, many keys" (cache bytes) and the
  "Inference Lab increment" list (attention_flops, score_bytes, kv_bytes,
  fit_exponent).
* "E8.1 IO-aware attention" (coursefy.online), "Do it in code" (score_bytes,
  tile_bytes, num_blocks) and the chapter reference's traffic lower bound
  t >= M_read / BW.
"""

from __future__ import annotations

import math

import numpy as np


def causal_pairs(q_len: int, kv_len: int) -> int:
    """Number of visible (query, key) pairs under the causal rule.

    Query i sees keys j <= i + (kv_len - q_len).  For self-attention
    (q_len == kv_len == T) this is T(T+1)/2 ("What is being computed":
    position i sees i keys counting itself).
    """
    if q_len > kv_len:
        raise ValueError("causal needs q_len <= kv_len")
    off = kv_len - q_len
    # rows i = 0..q_len-1 see min(kv_len, i + off + 1) = i + off + 1 keys
    return q_len * (off + 1) + q_len * (q_len - 1) // 2


def attention_flops(batch: int, heads: int, q_len: int, kv_len: int, head_dim: int,
                    causal: bool = False) -> int:
    """4 * B * h * d * (number of pairs): two products of 2 flops per
    multiply-add over every visible (query, key) pair.

    "Attention and Its Computational Cost", "What is being computed": each
    product costs 2 T_q T_kv d; the chapter's evidence table gives the total
    4 B h T_q T_kv d, with causal counting T(T+1)/2 pairs.
    """
    pairs = causal_pairs(q_len, kv_len) if causal else q_len * kv_len
    return 4 * batch * heads * head_dim * pairs


def score_bytes(n: int, bytes_per_value: int = 2) -> int:
    """Size of one full n x n score matrix ("E8.1", "Do it in code")."""
    return n * n * bytes_per_value


def score_tensor_bytes(seq_len: int, heads: int, bytes_per_value: int = 2, batch: int = 1) -> int:
    """One T x T score tensor over all heads of a batch
    ("The cost of writing down the scores", score-size table)."""
    return batch * heads * score_bytes(seq_len, bytes_per_value)


def tile_bytes(t: int, bytes_per_value: int = 2) -> int:
    """Size of one t x t tile ("E8.1", "Do it in code")."""
    return t * t * bytes_per_value


def num_blocks(n: int, block: int) -> int:
    """ceil(n / block); block must be >= 1 ("E8.1", "Do it in code")."""
    if block < 1:
        raise ValueError("block must be at least 1")
    return -(-n // block)


def kv_bytes(layers: int, heads: int, head_dim: int, seq_len: int, bytes_per_value: int = 2,
             batch: int = 1) -> int:
    """Bytes of cached keys plus values: 2 * layers * heads * d * T * bytes,
    per sequence, times the batch.

    The formula on "Attention and Its Computational Cost", section "The other
    shape: one query, many keys" did not survive extraction; this reading
    reproduces its printed totals (36 MiB at 1,024 tokens and 144 MiB at 4,096
    for 12 layers of 12 heads of 64 in fp16) and the one-layer cache-read
    column of its decode timing table.
    """
    return 2 * layers * heads * head_dim * seq_len * bytes_per_value * batch


def fit_exponent(xs, ys) -> float:
    """Least-squares slope of log(y) against log(x): the power-law exponent
    ("Attention and Its Computational Cost", section "Time": fitted exponents
    of the timing table for T >= 1,024)."""
    lx = np.log(np.asarray(xs, dtype=np.float64))
    ly = np.log(np.asarray(ys, dtype=np.float64))
    dx = lx - lx.mean()
    return float((dx * (ly - ly.mean())).sum() / (dx * dx).sum())


def min_transfer_time(bytes_moved: float, bandwidth: float) -> float:
    """Traffic lower bound t >= M_read / BW ("E8.1", chapter reference, "Math
    and notation" and its worked example)."""
    if bandwidth <= 0 or not math.isfinite(bandwidth):
        raise ValueError("bandwidth must be positive and finite")
    return bytes_moved / bandwidth
