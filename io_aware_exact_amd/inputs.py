"""Seeded synthetic inputs for attention workloads.

This module is shared by the GPU tests, the benchmark and the oracle checks,
so it holds none of the attention arithmetic: only random draws, the optional
spread factor applied to K, and rounding to the storage dtype.

Recipe (the pages' workloads are random N(0,1) tensors at GPT-2's head shape
and at the sizes listed in ``WORKLOADS``):

* tensor ``t`` in (q=0, k=1, v=2), batch row ``b``: draw
  ``numpy.random.default_rng([seed, t, b]).standard_normal((H, T, d), float32)``
  (H is the number of key/value heads for k and v);
* multiply by the tensor's factor in float32 (K x 3 for the mid-length
  workload, 1 otherwise);
* round to bfloat16 by round-to-nearest-even (torch's float32 -> bfloat16
  cast), or keep float32.

Seeding per (tensor, batch row) lets a test regenerate one batch row of a
large workload without drawing the rest, and lets rows be drawn in parallel
threads (numpy releases the GIL while filling).
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np
import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Tq: int
    Tkv: int
    d: int
    dtype: str          # "bf16" or "f32"
    causal: bool
    seed: int
    k_factor: float = 1.0
    num_splits: int = 1
    block: int = 64
    Hkv: int | None = None   # key/value heads (grouped-query); None = H

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def kv_heads(self) -> int:
        return self.H if self.Hkv is None else self.Hkv

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # exact check: fp32, one head, 256 x 256, d=64, key block 64
    "tiny": Workload("tiny", 1, 1, 256, 256, 64, "f32", False, seed=1),
    # GPT-2-shaped prefill
    "gpt2": Workload("gpt2", 4, 12, 1024, 1024, 64, "bf16", True, seed=2),
    # mid-length prefill, K rows scaled by 3 to spread the scores
    "mid": Workload("mid", 2, 16, 4096, 4096, 64, "bf16", False, seed=3, k_factor=3.0),
    "mid_causal": Workload("mid_causal", 2, 16, 4096, 4096, 64, "bf16", True, seed=3, k_factor=3.0),
    # the mid-length prefill at head width 128
    "mid_d128": Workload("mid_d128", 2, 16, 4096, 4096, 128, "bf16", False, seed=10, k_factor=3.0),
    "mid_d128_causal": Workload("mid_d128_causal", 2, 16, 4096, 4096, 128, "bf16", True, seed=10, k_factor=3.0),
    # long-context causal prefill
    "long": Workload("long", 1, 12, 16384, 16384, 64, "bf16", True, seed=4),
    # one head of a 16K-token sequence (batch 1): too few query tiles to fill
    # the chip, the case for splitting the key axis of prefill
    "long_1head": Workload("long_1head", 1, 1, 16384, 16384, 64, "bf16", True, seed=7),
    "long_1head_full": Workload("long_1head_full", 1, 1, 16384, 16384, 64, "bf16", False, seed=8),
    # one query per sequence against 8,192 cached keys, split-KV into 16 chunks
    "decode": Workload("decode", 64, 32, 1, 8192, 128, "bf16", False, seed=5, num_splits=16),
    # one sequence of GPT-2's head shape against 16,384 cached keys (batch 1):
    # the library picks the number of key partitions
    "decode_b1": Workload("decode_b1", 1, 12, 1, 16384, 64, "bf16", False, seed=9, num_splits=0),
    # the same decode step with grouped-query attention: 32 query heads over
    # 8 key/value heads (groups of 4), so a quarter of the cache
    "decode_gqa": Workload("decode_gqa", 64, 32, 1, 8192, 128, "bf16", False, seed=6, num_splits=16, Hkv=8),
}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_rows(seed: int, tensor: str, b: int, shape, factor: float = 1.0) -> np.ndarray:
    """float32 N(0,1) draws for one batch row of one tensor, times ``factor``."""
    rng = np.random.default_rng([seed, TENSOR_IDS[tensor], b])
    x = rng.standard_normal(tuple(shape), dtype=np.float32)
    if factor != 1.0:
        x *= np.float32(factor)
    return x


def _torch_dtype(dtype: str):
    if dtype == "bf16":
        return torch.bfloat16
    if dtype == "f32":
        return torch.float32
    raise ValueError(f"unknown dtype {dtype!r}")


def make_tensor(seed: int, tensor: str, B: int, H: int, T: int, d: int, dtype: str,
                factor: float = 1.0, batch_rows=None) -> torch.Tensor:
    """A contiguous CPU tensor [B', H, T, d] in ``dtype``.

    ``batch_rows`` selects which batch rows to draw (default: all B); the
    result then holds only those rows, in the given order, with values equal
    to the same rows of the full tensor.
    """
    rows = list(range(B)) if batch_rows is None else [int(r) for r in batch_rows]
    out = torch.empty((len(rows), H, T, d), dtype=_torch_dtype(dtype))

    def fill(i):
        x = normal_rows(seed, tensor, rows[i], (H, T, d), factor)
        out[i].copy_(torch.from_numpy(x))   # float32 -> bf16 cast rounds to nearest even

    if len(rows) == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(len(rows))))
    return out


def make_qkv(w: Workload, batch_rows=None):
    """(q, k, v) CPU tensors for a workload (see the module recipe)."""
    q = make_tensor(w.seed, "q", w.B, w.H, w.Tq, w.d, w.dtype, 1.0, batch_rows)
    k = make_tensor(w.seed, "k", w.B, w.kv_heads, w.Tkv, w.d, w.dtype, w.k_factor, batch_rows)
    v = make_tensor(w.seed, "v", w.B, w.kv_heads, w.Tkv, w.d, w.dtype, 1.0, batch_rows)
    return q, k, v


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a (bf16 or fp32) tensor, on the host."""
    return t.detach().to("cpu").to(torch.float64).numpy()
