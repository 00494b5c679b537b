"""The entry points inside HIP graph capture.

The library allocates nothing, issues no memset, copy or synchronisation and
takes every buffer from the caller, so its calls can be captured into a
graph and replayed.  Each test captures one call with static buffers, then
replays it several times with new inputs copied in eagerly between replays
(plus an eager call and a synchronisation of the program's own), and checks
every replay against an eager call on the same inputs.  The kernels are
deterministic (no atomics, fixed reduction order), so the comparison is
bitwise.
"""

import sys

import pytest
import torch

import io_aware_exact_amd as attn

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

REPLAYS = 3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rand(shape, seed, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype)


def capture(prepare):
    """Capture prepare()() (the call built on the capture stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        prepare()()                      # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        prepare()()
    return graph


@pytest.mark.parametrize("B,H,T,d,causal", [(2, 4, 300, 64, True), (1, 3, 200, 128, False), (8, 96, 129, 64, True),
                                            (4, 100, 129, 64, False)])
def test_graph_replay_prefill(B, H, T, d, causal):
    say(f"case prefill B={B} H={H} T={T} d={d} causal={causal}")
    q, k, v = (torch.empty(B, H, T, d, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, T, dtype=torch.float32, device="cuda")
    for t in (q, k, v):
        t.copy_(rand(t.shape, 1))
    graph = capture(lambda: attn.prepared_fwd(q, k, v, o, lse, causal))
    for rep in range(REPLAYS):
        for i, t in enumerate((q, k, v)):
            t.copy_(rand(t.shape, 100 * rep + i))
        graph.replay()
        torch.cuda.synchronize()
        o_g, lse_g = o.clone(), lse.clone()
        o_e, lse_e = attn.attn_fwd(q, k, v, causal=causal)
        torch.cuda.synchronize()
        say(f"  replay {rep}: kernel {attn.attn_last_kernel()}")
        assert torch.equal(o_g, o_e) and torch.equal(lse_g, lse_e)


def test_graph_replay_split_prefill():
    B, H, T, d = 1, 1, 4096, 64
    say(f"case split prefill B={B} H={H} T={T} d={d} causal")
    q, k, v = (torch.empty(B, H, T, d, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, T, dtype=torch.float32, device="cuda")
    ws = torch.empty(attn.attn_fwd_split_workspace_bytes(B, H, T, T, d, True, 0), dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0
    for t in (q, k, v):
        t.copy_(rand(t.shape, 2))
    graph = capture(lambda: attn.prepared_fwd(q, k, v, o, lse, True, kv_chunk=0, workspace=ws))
    for rep in range(REPLAYS):
        for i, t in enumerate((q, k, v)):
            t.copy_(rand(t.shape, 200 + 100 * rep + i))
        graph.replay()
        torch.cuda.synchronize()
        o_g, lse_g = o.clone(), lse.clone()
        o_e, lse_e = attn.attn_fwd_split(q, k, v, causal=True, kv_chunk=0)
        torch.cuda.synchronize()
        say(f"  replay {rep}: kernel {attn.attn_last_kernel()}")
        assert "combine" in attn.attn_last_kernel()
        assert torch.equal(o_g, o_e) and torch.equal(lse_g, lse_e)


@pytest.mark.parametrize("Hkv,splits", [(32, 16), (8, 16), (32, 0)])
def test_graph_replay_decode(Hkv, splits):
    B, Hq, T, d = 4, 32, 2048, 128
    say(f"case decode B={B} Hq={Hq} Hkv={Hkv} T={T} d={d} splits={splits}")
    q = torch.empty(B, Hq, 1, d, dtype=torch.bfloat16, device="cuda")
    k, v = (torch.empty(B, Hkv, T, d, dtype=torch.bfloat16, device="cuda") for _ in range(2))
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    p = splits or attn.attn_decode_splits(B, Hq, Hkv, T, d)
    ws = torch.empty(max(16, attn.attn_decode_workspace_bytes(B, Hq, d, p)), dtype=torch.uint8, device="cuda")
    for t in (q, k, v):
        t.copy_(rand(t.shape, 3))
    graph = capture(lambda: attn.prepared_decode(q, k, v, o, lse, splits, ws))
    for rep in range(REPLAYS):
        for i, t in enumerate((q, k, v)):
            t.copy_(rand(t.shape, 300 + 100 * rep + i))
        graph.replay()
        torch.cuda.synchronize()
        o_g, lse_g = o.clone(), lse.clone()
        o_e, lse_e = attn.attn_decode_gqa(q, k, v, num_splits=splits)
        torch.cuda.synchronize()
        say(f"  replay {rep}: kernel {attn.attn_last_kernel()}")
        assert torch.equal(o_g, o_e) and torch.equal(lse_g, lse_e)


@pytest.mark.parametrize("d", [64, 128])
def test_graph_replay_backward(d):
    B, H, T = 2, 4, 384
    say(f"case backward B={B} H={H} T={T} d={d} causal")
    q, k, v, do = (torch.empty(B, H, T, d, dtype=torch.bfloat16, device="cuda") for _ in range(4))
    for i, t in enumerate((q, k, v, do)):
        t.copy_(rand(t.shape, 40 + i))
    o, lse = attn.attn_fwd(q, k, v, causal=True)
    gq, gk, gv = (torch.empty(B, H, T, d, dtype=torch.float32, device="cuda") for _ in range(3))
    ws = torch.empty(attn.attn_bwd_workspace_bytes(B, H, T), dtype=torch.uint8, device="cuda")
    graph = capture(lambda: attn.prepared_bwd(q, k, v, o, lse, do, gq, gk, gv, True, ws))
    for rep in range(REPLAYS):
        do.copy_(rand(do.shape, 500 + rep))
        graph.replay()
        torch.cuda.synchronize()
        got = (gq.clone(), gk.clone(), gv.clone())
        ref = attn.attn_bwd(q, k, v, o, lse, do, causal=True)
        torch.cuda.synchronize()
        say(f"  replay {rep}: kernel {attn.attn_last_kernel()}")
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
