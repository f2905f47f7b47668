"""Capture of the library's launches into a HIP graph (torch.cuda.graph).

The entry points allocate nothing and enqueue no memset, only kernels on the
caller's stream, so a caller can capture them (a serving loop, for one).
Each test runs the call eagerly once (which also sets the kernels' LDS
attributes), captures the same call into a graph, and replays the graph
several times with eager work and synchronisations between the replays; the
outputs are overwritten with NaN before every replay and must come back
bitwise equal to the eager result (the kernels are deterministic).
"""

import pytest
import torch

from workloads import make_qkv

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _check_replays(graph, outs, refs, n=4):
    for i in range(n):
        for o in outs:
            o.fill_(float("nan"))
        x = torch.randn(4096, device="cuda")  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        y = (x * 2).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(y)
        for o, r in zip(outs, refs):
            assert torch.equal(o, r), f"replay {i} differs from the eager result"


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("case", [(2, 4, 1000, 128, torch.bfloat16, False),
                                  (2, 32, 1100, 128, torch.bfloat16, True),  # persistent launch
                                  (1, 2, 300, 64, torch.float32, True)],
                         ids=["bf16-d128", "bf16-d128-causal-persistent", "fp32-d64-causal"])
def test_fwd_graph_replays(gpu_lib, case):
    B, H, N, d, dt, causal = case
    _say(f"[graph] fa_fwd B={B} H={H} N={N} d={d} {dt} causal={causal}")
    q, k, v = make_qkv(B, H, N, d, dt, seed=7, device="cuda")
    O = torch.empty_like(q)
    L = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    call = lambda: gpu_lib.fwd(q, k, v, causal=causal, out=O, lse=L)
    call()
    torch.cuda.synchronize()
    refs = (O.clone(), L.clone())
    g = _capture(call)
    _check_replays(g, (O, L), refs)


def test_splitkv_graph_replays(gpu_lib):
    B, H, N, d, S = 1, 2, 3000, 128, 4
    _say(f"[graph] fa_fwd_splitkv B={B} H={H} N={N} d={d} splits={S}")
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, seed=8, device="cuda")
    O = torch.empty_like(q)
    L = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(gpu_lib.fa_fwd_splitkv_workspace(B, H, N, d, S), dtype=torch.uint8,
                     device="cuda")
    call = lambda: gpu_lib.fwd_splitkv(q, k, v, S, causal=True, out=O, lse=L, workspace=ws)
    call()
    torch.cuda.synchronize()
    refs = (O.clone(), L.clone())
    g = _capture(call)
    _check_replays(g, (O, L), refs)


def test_bwd_graph_replays(gpu_lib):
    B, H, N, d = 1, 4, 700, 64
    _say(f"[graph] fa_bwd B={B} H={H} N={N} d={d} causal")
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, seed=9, device="cuda")
    do = make_qkv(B, H, N, d, torch.bfloat16, seed=10, device="cuda")[0]
    O, L = gpu_lib.fwd(q, k, v, causal=True)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(gpu_lib.fa_bwd_workspace(B, H, N, d), dtype=torch.uint8, device="cuda")
    call = lambda: gpu_lib.bwd(q, k, v, O, do, L, causal=True, dq=dq, dk=dk, dv=dv,
                               workspace=ws)
    call()
    torch.cuda.synchronize()
    refs = (dq.clone(), dk.clone(), dv.clone())
    g = _capture(call)
    _check_replays(g, (dq, dk, dv), refs)
