"""Pins of the oracle's cost model against figures printed on the pages."""

import json
import math
import os

import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MiB = 1024 ** 2
GiB = 1024 ** 3


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_lesson_constants():
    g = _load("lesson_constants.json")["lesson"]
    assert oracle.score_bytes(g["n"], g["bytes_per_value"]) == g["score_matrix_MiB"] * MiB
    assert oracle.tile_bytes(g["tile"], g["bytes_per_value"]) == g["tile_bytes"]
    assert oracle.num_blocks(g["n"], g["tile"]) == g["blocks_per_row"]
    assert oracle.num_blocks(4097, 128) == 33
    assert oracle.num_blocks(1, 1) == 1


def test_score_tensor_table():
    g = _load("score_tensor_sizes.json")
    for row in g["rows"]:
        b = oracle.score_tensor_bytes(row["T"], g["heads"], g["bytes_per_value"])
        unit = MiB if row["unit"] == "MiB" else GiB
        # the page prints one decimal for GiB rows and whole MiB otherwise
        assert round(b / unit, 1) == row["value"]


def test_memory_efficient_peak_is_output_size():
    g = _load("memory_efficient_peak.json")
    for row in g["rows"]:
        out = g["heads"] * row["T"] * g["head_dim"] * g["bytes_per_value"]
        assert round(out / MiB) == row["printed_MiB"] or (row["T"] == 512 and out / MiB < 1.0)
    # the 16,384 row is exact
    assert 12 * 16384 * 64 * 2 == 24 * MiB


def test_tiling_article_constants():
    g = _load("lesson_constants.json")["tiling_article"]
    it = g["intermediate"]
    assert it["heads"] * oracle.score_bytes(it["n"], it["bytes_per_value"]) == it["printed_MiB"] * MiB
    acc = g["accumulator"]
    assert acc["B_q"] * acc["d_v"] * acc["bytes_per_value"] == acc["printed_KiB"] * 1024
    qb = g["query_blocks"]
    assert oracle.num_blocks(qb["n"], qb["B_q"]) == qb["count"]
    lc = g["long_context_kv"]
    kv = oracle.kv_bytes(1, 1, lc["d_model"], lc["positions"], lc["bytes_per_value"])
    assert round(kv / GiB) == lc["printed_GiB"]
    # four passes over n^2 16-bit elements against 4 n^2 d flops -> d/2 flop/B
    ins = g["intensity"]
    n = 4096
    flops = oracle.attention_flops(1, 1, n, n, ins["d_k"])
    assert flops / (4 * oracle.score_bytes(n, 2)) == ins["flops_per_byte"]


def test_traffic_bound_worked_example():
    g = _load("lesson_constants.json")["traffic_bound"]
    t = oracle.min_transfer_time(g["weights_GB"] * 1e9, g["bandwidth_GBps"] * 1e9)
    assert math.isclose(t, g["seconds"])
    assert math.isclose(1.0 / t, g["steps_per_second"])
    t2 = oracle.min_transfer_time(g["kv_MiB"] * MiB, g["link_GiBps"] * GiB)
    assert math.isclose(t2, g["kv_seconds"])
    with pytest.raises(ValueError):
        oracle.min_transfer_time(1.0, 0.0)


def test_kv_cache_table():
    g = _load("kv_cache_table.json")
    for row in g["per_sequence"]:
        b = oracle.kv_bytes(g["layers"], g["heads"], g["head_dim"], row["T"], g["bytes_per_value"])
        assert b == row["printed_MiB"] * MiB
    for row in g["rows"]:
        b = oracle.kv_bytes(g["layers"], g["heads"], g["head_dim"], row["T"], g["bytes_per_value"], row["batch"])
        if row["unit"] == "MiB":
            assert b == row["value"] * MiB
        else:
            # printed to one decimal, rounding half up (2.25 GiB -> "2.3 GiB")
            assert math.floor(b / GiB * 10 + 0.5) / 10 == row["value"]
        assert round(100 * b / (g["weights_MB"] * 1e6)) == row["percent_of_weights"]
    f = g["decode_flops"]
    flops = oracle.attention_flops(1, f["heads"], 1, f["T"], f["head_dim"])
    assert 2.9e6 < flops < 3.3e6          # "about three million"
    assert flops == 4 * f["heads"] * f["T"] * f["head_dim"]


def test_decode_table_bytes_and_bandwidth():
    g = _load("decode_table.json")
    for row in g["rows"]:
        b = oracle.kv_bytes(g["layers"], g["heads"], g["head_dim"], row["T"], g["bytes_per_value"], row["batch"])
        mib = b / MiB
        assert round(mib, 1 if mib < 1 else 0) == row["cache_MiB"]
        gbps = b / (row["time_us"] * 1e-6) / 1e9
        assert round(gbps) == row["GBps"]
        # and the time is the traffic bound at that bandwidth
        assert oracle.min_transfer_time(b, gbps * 1e9) == pytest.approx(row["time_us"] * 1e-6)


def test_timing_table_throughput_and_exponents():
    g = _load("timing_table.json")
    T = g["T"]
    # causal-counted throughput of the efficient fp16 kernel at 8,192
    fl = oracle.attention_flops(1, g["heads"], 8192, 8192, g["head_dim"], causal=True)
    assert fl == 4 * 12 * 64 * 8192 * 8193 // 2
    t8192 = g["fp16_efficient_ms"][T.index(8192)] * 1e-3
    assert round(fl / t8192 / 1e12, 1) == g["efficient_fp16_TFLOPs"]["8192"]
    # at 1,024 the printed 11.7 TFLOP/s implies a time that rounds to the printed 0.14 ms
    fl1 = oracle.attention_flops(1, 12, 1024, 1024, 64, causal=True)
    assert round(fl1 / (g["efficient_fp16_TFLOPs"]["1024"] * 1e12) * 1e3, 2) == 0.14
    # naive at 8,192: about 1.5 TFLOP/s on the causal count
    tn = g["fp16_naive_ms"][T.index(8192)] * 1e-3
    assert round(fl / tn / 1e12, 1) == g["naive_fp16_TFLOPs_8192"]
    # exponents for T >= 1,024; the page's inputs are rounded, allow 0.015
    sel = [i for i, t in enumerate(T) if t >= 1024]
    for key, want in g["fitted_exponent_T_ge_1024"].items():
        ys = [g[f"{key}_ms"][i] for i in sel]
        got = oracle.fit_exponent([T[i] for i in sel], ys)
        assert abs(got - want) <= 0.015, (key, got, want)
    assert oracle.fit_exponent([1, 2, 4, 8], [3, 12, 48, 192]) == pytest.approx(2.0, abs=1e-12)
    est = g["naive_traffic_estimate"]
    elems = oracle.score_tensor_bytes(est["T"], 12, 1)
    assert round(elems / 1e6) == est["elements_million"]
    assert round(elems * est["bytes_per_element"] / 1e9, 1) == est["GB"]
    assert round(oracle.min_transfer_time(elems * 12, est["copy_GBps"] * 1e9) * 1e3) == est["ms"]


def test_flops_doubling_properties():
    """Doubling the prompt quadruples prefill FLOPs; doubling the cache doubles
    decode FLOPs ("What is being computed", shapes table)."""
    for T in (64, 1000, 4096):
        assert oracle.attention_flops(2, 3, 2 * T, 2 * T, 64) == 4 * oracle.attention_flops(2, 3, T, T, 64)
        assert oracle.attention_flops(2, 3, 1, 2 * T, 64) == 2 * oracle.attention_flops(2, 3, 1, T, 64)
    assert oracle.causal_pairs(5, 5) == 15
    assert oracle.causal_pairs(1, 9) == 9
    assert oracle.causal_pairs(3, 5) == 3 + 4 + 5
    brute = sum(1 for i in range(7) for j in range(11) if j <= i + 4)
    assert oracle.causal_pairs(7, 11) == brute
    with pytest.raises(ValueError):
        oracle.causal_pairs(6, 5)
