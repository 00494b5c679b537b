"""The seeded input recipe: deterministic, row-addressable, correctly rounded."""

import numpy as np
import torch

from io_aware_exact_amd.inputs import WORKLOADS, make_qkv, make_tensor, normal_rows, to_f64


def test_rows_are_reproducible_and_addressable():
    full = make_tensor(9, "k", 4, 2, 8, 16, "bf16", 3.0)
    part = make_tensor(9, "k", 4, 2, 8, 16, "bf16", 3.0, batch_rows=[2, 0])
    assert torch.equal(part[0], full[2]) and torch.equal(part[1], full[0])
    again = make_tensor(9, "k", 4, 2, 8, 16, "bf16", 3.0)
    assert torch.equal(full, again)


def test_bf16_is_round_to_nearest_even_of_the_fp32_draw():
    x = normal_rows(3, "q", 1, (2, 5, 8))
    t = make_tensor(3, "q", 2, 2, 5, 8, "bf16")[1]
    bits = x.view(np.uint32).astype(np.uint64)
    # RNE on the upper 16 bits, written out on the bit pattern
    lower = bits & 0xFFFF
    upper = bits >> 16
    up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    rounded = ((upper + up.astype(np.uint64)) << 16).astype(np.uint32).view(np.float32)
    np.testing.assert_array_equal(to_f64(t), rounded.astype(np.float64))


def test_streams_differ_between_tensors_and_rows():
    a = normal_rows(2, "q", 0, (4,))
    b = normal_rows(2, "k", 0, (4,))
    c = normal_rows(2, "q", 1, (4,))
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_workload_shapes():
    w = WORKLOADS["tiny"]
    q, k, v = make_qkv(w)
    assert q.dtype == torch.float32 and q.shape == (1, 1, 256, 64)
    assert w.scale == 1.0 / 8.0
    d = WORKLOADS["decode"]
    assert (d.B, d.H, d.Tq, d.Tkv, d.d, d.num_splits) == (64, 32, 1, 8192, 128, 16)
    m = WORKLOADS["mid"]
    q, k, v = make_qkv(m.with_(B=1, H=1, Tq=8, Tkv=8))
    assert abs(float(k.float().std()) - 3.0) < 1.5
