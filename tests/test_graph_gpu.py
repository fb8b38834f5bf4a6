"""The library's launches inside a captured HIP graph.

Every entry point only enqueues kernels on the caller's stream (no
allocation, no synchronisation, no memset), so a caller can capture it in a
graph and replay it.  Each test captures calls with preallocated outputs,
replays the graph several times with eager work and synchronisations between
the replays, and checks every replay bit for bit against the eager result
(new inputs are copied into the captured input buffers between replays).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import io_aware_exact_03_amd as fa  # noqa: E402
from workloads import random_qkv  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs(B, H, Hkv, N, d, seed):
    q, _, _, rng = random_qkv(B, H, N, d, seed, "bf16")
    _, k, v, rng = random_qkv(B, Hkv, N, d, seed + 1, "bf16", rng=rng)
    do = rng.standard_normal(q.shape).astype(np.float32)
    return [torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (q, k, v, do)]


def _replay_and_check(graph, bufs, outs, eager, seeds, make):
    """For each seed: copy fresh inputs into the captured buffers, replay,
    run some unrelated eager work and a synchronisation, compare with the
    eager computation on the same inputs."""
    for seed in seeds:
        fresh = make(seed)
        for b, x in zip(bufs, fresh):
            b.copy_(x)
        graph.replay()
        junk = torch.randn(1 << 20, device="cuda").cumsum(0)  # eager work in between
        torch.cuda.synchronize()
        ref = eager(*fresh)
        for got, want in zip(outs, ref):
            assert torch.equal(got, want), f"replay with seed {seed} differs from eager"
        del junk


@pytest.mark.parametrize("causal", [False, True])
def test_forward_in_graph(causal):
    B, H, N, d = 2, 4, 700, 128
    make = lambda s: _inputs(B, H, H, N, d, s)[:3]
    q, k, v = make(1)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fwd(q, k, v, causal=causal, out=o, lse=lse)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fwd(q, k, v, causal=causal, out=o, lse=lse)

    def eager(q2, k2, v2):
        return fa.fwd(q2, k2, v2, causal=causal)
    _replay_and_check(g, [q, k, v], [o, lse], eager, [2, 3, 4], make)


def test_split_forward_in_graph():
    B, H, N, d = 1, 2, 3000, 128
    need = fa.fa_fwd_workspace_size(B, H, N, d, fa.DTYPE_BF16)
    assert need > 0
    make = lambda s: _inputs(B, H, H, N, d, s)[:3]
    q, k, v = make(5)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fwd(q, k, v, causal=True, out=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fwd(q, k, v, causal=True, out=o, lse=lse, workspace=ws)
    ws_eager = torch.empty_like(ws)

    def eager(q2, k2, v2):
        return fa.fwd(q2, k2, v2, causal=True, workspace=ws_eager)
    _replay_and_check(g, [q, k, v], [o, lse], eager, [6, 7, 8], make)


@pytest.mark.parametrize("H_kv,use_ws", [(4, True), (1, True), (4, False)])
def test_backward_in_graph(H_kv, use_ws):
    # on this small grid the workspace brings in the dK/dV and dQ splits
    B, H, N, d = 1, 4, 500, 64
    make = lambda s: _inputs(B, H, H_kv, N, d, s)
    q, k, v, do = make(9)
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty_like(lse)
    need = fa.fa_bwd_workspace_size(B, H, H_kv, N, d)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if use_ws else None

    def step():
        fa.fwd(q, k, v, causal=True, out=o, lse=lse)
        fa.bwd(q, k, v, o, do, lse, causal=True, dq=dq, dk=dk, dv=dv, delta=delta, workspace=ws)
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    ws_eager = torch.empty_like(ws) if use_ws else None

    def eager(q2, k2, v2, do2):
        o2, l2 = fa.fwd(q2, k2, v2, causal=True)
        return (o2, l2) + fa.bwd(q2, k2, v2, o2, do2, l2, causal=True, workspace=ws_eager)
    _replay_and_check(g, [q, k, v, do], [o, lse, dq, dk, dv], eager, [10, 11, 12], make)
