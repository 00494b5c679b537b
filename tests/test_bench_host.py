"""Host logic of bench.py (no GPU).

The refusal of more than one GPU, the algorithmic flop and byte counts the
roofline divides by (against the cost model and brute force), the digest of
the device sources, and the rule that recorded HBM traffic is reported only
while it was taken on the current device sources and on the kernel that ran.
"""

import importlib.util
import json
import os
import shutil
import subprocess
import sys

import pytest

from io_aware_exact_amd.inputs import WORKLOADS
from oracle import cost

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


bench = load_bench()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert r.stdout == ""                      # no JSON line
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("tq,tkv", [(1, 1), (1, 7), (5, 5), (3, 9), (8, 64), (17, 40)])
@pytest.mark.parametrize("causal", [False, True])
def test_visible_pairs_brute_force(tq, tkv, causal):
    # query i sees key j when j <= i + (tkv - tq) (bottom-right causal alignment)
    want = sum(1 for i in range(tq) for j in range(tkv) if not causal or j <= i + tkv - tq)
    assert bench.visible_pairs(tq, tkv, causal) == want


@pytest.mark.parametrize("name", sorted(n for n, w in WORKLOADS.items() if w.Tq > 1))
def test_prefill_flops_match_cost_model(name):
    w = WORKLOADS[name]
    assert bench.prefill_flops(w) == cost.attention_flops(w.B, w.H, w.Tq, w.Tkv, w.d, w.causal)


def test_headline_counts():
    w = WORKLOADS["gpt2"]
    assert bench.prefill_flops(w) == 4 * 4 * 12 * 64 * (1024 * 1025 // 2)      # 6.45 GFLOP
    # Q, K, V, O in bf16 and the fp32 LSE, each once
    assert bench.prefill_bytes(w) == 4 * 12 * (4 * 1024 * 64 * 2 + 1024 * 4) == 25_362_432
    total, kv = bench.decode_bytes(WORKLOADS["decode"])
    assert kv == 8 * 2 ** 30 == cost.kv_bytes(1, 32, 128, 8192, batch=64)
    assert total == kv + 2 * 64 * 32 * 128 * 2 + 64 * 32 * 4
    # grouped-query: the cache of 8 key/value heads, q / O / LSE of 32
    total_g, kv_g = bench.decode_bytes(WORKLOADS["decode_gqa"])
    assert kv_g == kv // 4 and total_g - kv_g == total - kv


def copy_sources(dst):
    src = os.path.join(ROOT, "io_aware_exact_amd", "csrc")
    os.makedirs(os.path.join(dst, "io_aware_exact_amd"))
    shutil.copytree(src, os.path.join(dst, "io_aware_exact_amd", "csrc"))
    return os.path.join(dst, "io_aware_exact_amd", "csrc")


def test_digest_ignores_comments_not_code(tmp_path, monkeypatch):
    csrc = copy_sources(str(tmp_path))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_sources_digest()
    assert base == load_bench().kernel_sources_digest()   # same text, same digest
    path = os.path.join(csrc, "decode.hip")
    with open(path) as f:
        text = f.read()
    with open(path, "w") as f:
        f.write("// a new comment\n/* and a block\n   comment */\n" + text.replace("\n", "\n\n", 3))
    assert bench.kernel_sources_digest() == base
    with open(path, "w") as f:
        f.write(text + "\nstatic int extra_symbol = 1;\n")
    assert bench.kernel_sources_digest() != base


def test_traffic_reported_only_for_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    kern = "prefill_bf16_d64<waves=4,bq=64,bk=64,key_halves=2,stages=2,causal>"
    assert bench.measured_traffic("prefill", "gpt2", kern) is None          # no record
    rec = {"gpt2": {"prefill": {"sources_sha256_16": bench.kernel_sources_digest(), "kernel": kern,
                                "fetch_bytes": 1000.4, "write_bytes": 24.0}}}
    with open(os.path.join(tmp_path, "traffic.json"), "w") as f:
        json.dump(rec, f)
    assert bench.measured_traffic("prefill", "gpt2", kern) == 1024
    assert bench.measured_traffic("decode", "gpt2", kern) is None
    # counted on another kernel than the one that ran
    assert bench.measured_traffic("prefill", "gpt2", kern.replace("stages=2", "stages=3")) is None
    rec["gpt2"]["prefill"]["sources_sha256_16"] = "0" * 16
    with open(os.path.join(tmp_path, "traffic.json"), "w") as f:
        json.dump(rec, f)
    assert bench.measured_traffic("prefill", "gpt2", kern) is None          # taken on other sources


def test_digest_covers_device_code_only(tmp_path, monkeypatch):
    csrc = copy_sources(str(tmp_path))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_sources_digest()
    with open(os.path.join(csrc, "api.cpp"), "a") as f:          # host-side checks
        f.write("\nstatic int extra_check = 1;\n")
    assert bench.kernel_sources_digest() == base
    with open(os.path.join(csrc, "common.hpp"), "a") as f:       # shared by the kernels
        f.write("\nstatic int extra_symbol = 1;\n")
    assert bench.kernel_sources_digest() != base


def test_committed_counters_were_taken_on_these_sources():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    digest = bench.kernel_sources_digest()
    entries = [(wl, k, e) for wl, by in rec.items() if isinstance(by, dict)
               for k, e in by.items() if isinstance(e, dict) and "sources_sha256_16" in e]
    assert entries
    stale = [(wl, k) for wl, k, e in entries if e["sources_sha256_16"] != digest]
    assert not stale, f"HBM counters recorded on other kernel sources: {stale}"


def test_mfma_probe_library_exports():
    import ctypes

    path = os.path.join(ROOT, "io_aware_exact_amd", "libattn_probe.so")
    if not os.path.exists(path):
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(path)
    lib.probe_mfma_loop_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.probe_mfma_loop_flops.restype = ctypes.c_double
    lib.probe_mfma_loop_threads.restype = ctypes.c_int
    lib.probe_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.probe_mfma_loop_threads() == 256
    # blocks x 4 waves x iters x 4 MFMAs x (32*32*16*2) flops
    assert lib.probe_mfma_loop_flops(2048, 4096) == 2048 * 4 * 4096 * 4 * 32768
    assert lib.probe_mfma_loop(0, 1, None, None) != 0            # rejected before any launch
    assert lib.probe_mfma_loop(1, 1, None, None) != 0


def test_issue_probe_library_exports():
    import ctypes

    path = os.path.join(ROOT, "io_aware_exact_amd", "libattn_probe.so")
    if not os.path.exists(path):
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(path)
    lib.probe_issue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    bench = load_bench()
    assert lib.probe_issue_modes() == len(bench.ISSUE_MODES)
    assert lib.probe_issue_threads() == 256
    assert lib.probe_issue_operand_bytes() == 20 * 64 * 16     # 20 bf16x8 operands per lane
    # rejected before any launch: bad mode, occupancy outside 1..3, empty grid, null pointers
    one = ctypes.c_void_p(1)
    assert lib.probe_issue(6, 3, 1, 1, one, one, one, None) != 0
    assert lib.probe_issue(0, 4, 1, 1, one, one, one, None) != 0
    assert lib.probe_issue(0, 0, 1, 1, one, one, one, None) != 0
    assert lib.probe_issue(0, 3, 0, 1, one, one, one, None) != 0
    assert lib.probe_issue(0, 3, 1, 1, None, one, one, None) != 0


ROCMINFO_SAMPLE = """
*******
Agent 1
*******
  Name:                    Intel(R) Xeon(R) Platinum
  Max Clock Freq. (MHz):   3800
*******
Agent 2
*******
  Name:                    gfx950
  Marketing Name:          AMD Instinct MI355X
  Max Clock Freq. (MHz):   2400
"""


def test_rocminfo_clock_is_the_gpu_agents():
    assert bench.parse_rocminfo_clock(ROCMINFO_SAMPLE) == 2400
    assert bench.parse_rocminfo_clock("Name: gfx950\n") is None
    assert bench.parse_rocminfo_clock("") is None


def test_roofline_bound_follows_the_longer_time():
    # gpt2: 25.4 MB at 8 TB/s (3.17 us) outlasts 6.45 GFLOP at 2.5 PFLOP/s (2.58 us)
    r = bench.prefill_roofline(WORKLOADS["gpt2"], 0.01)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(25_362_432 / 1e-5 / 1e9)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0)
    for name in ("mid", "mid_causal", "long"):
        r = bench.prefill_roofline(WORKLOADS[name], 1.0)
        assert r["bound"] == "mfma" and r["peak"] == 2500.0
        assert r["achieved"] == pytest.approx(bench.prefill_flops(WORKLOADS[name]) / 1e-3 / 1e12)
    assert bench.prefill_roofline(WORKLOADS["tiny"], 1.0)["bound"] == "alu"


def test_headline_is_the_long_prefill():
    w = WORKLOADS[bench.HEADLINE]
    assert (w.B, w.H, w.Tq, w.Tkv, w.d, w.causal, w.dtype) == (1, 12, 16384, 16384, 64, True, "bf16")
    assert bench.prefill_flops(w) == 412_342_026_240          # 4 * 12 * 64 * 16384 * 16385 / 2


def test_leg_selection():
    import argparse
    ns = argparse.Namespace(no_decode=False, no_split=False, no_extra=False, no_backward=False)
    assert bench.parse_legs("all", ns) == list(bench.LEGS)
    assert bench.parse_legs("none", ns) == []
    assert bench.parse_legs("mid,mid_causal", ns) == ["mid", "mid_causal"]
    ns.no_decode = True
    assert not set(bench.parse_legs("all", ns)) & set(bench.DECODE_LEGS)
    with pytest.raises(SystemExit):
        bench.parse_legs("mid,nonsense", ns)


def test_sampled_rows_cover_edges_and_stay_in_range():
    import numpy as np
    rows = bench.sampled_rows(16384, 512, np.random.default_rng(0))
    assert rows.min() == 0 and rows.max() == 16383
    assert len(set(rows.tolist())) == rows.size >= 512
    assert {127, 128, 129, 16255, 16256} <= set(rows.tolist())
    small = bench.sampled_rows(40, 512, np.random.default_rng(0))
    assert small.tolist() == list(range(40))
