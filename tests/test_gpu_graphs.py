"""The forward entry points under HIP graph capture.

diffuser_attn and diffuser_attn_theta enqueue only kernel launches (and, at
K = 0, one device-to-device copy) on the caller's stream: no allocation, no
memset, no host synchronisation. A caller may therefore capture them in a
graph and replay it. Each case captures one call on fixed input and output
buffers, then replays it several times with new inputs copied in, eager
work and a synchronisation between the replays; every replay must equal an
eager call on the same inputs bit for bit (the kernels are deterministic).
The cases cover each forward route: the scheduled bf16 kernels at d = 64
and d = 32, the BigBird block-tile kernels, and the generic kernels in fp32.
"""
from __future__ import annotations

import pytest
import torch

import sparse_attention_hop_amd as sah
from workloads import make_tensor

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    # id, graph builder, B, H, d, dtype
    ("sched_d64", lambda: sah.build_graph(1100, 50, [0, 1, 2, 700, 1099], 40, 2, False, 3),
     2, 3, 64, torch.bfloat16),
    ("sched_d32", lambda: sah.build_graph(1024, 64, list(range(16)), 32, 1, True, 4),
     2, 2, 32, torch.bfloat16),
    ("block64", lambda: sah.build_block_graph(512, 64, 3, 3, 2, 1, 7), 2, 2, 64, torch.bfloat16),
    ("generic_f32", lambda: sah.build_graph(700, 20, [3, 400], 16, 1, False, 5),
     2, 2, 64, torch.float32),
]

REPLAYS = 3


def _inputs(shape, dtype, seed):
    return [make_tensor(shape, seed + i, dtype).to(DEV) for i in range(3)]


def _capture(fn):
    """Warm up on a side stream, then capture one call of fn."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def _replay_matches_eager(graph, bufs, out, shape, dtype, eager):
    for rep in range(REPLAYS):
        new = _inputs(shape, dtype, 1000 + 10 * rep)
        for dst, src in zip(bufs, new):
            dst.copy_(src)
        out.fill_(float("nan"))   # eager work between replays; the replay must overwrite it
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        expect = eager(*new)
        torch.cuda.synchronize()
        assert torch.equal(out, expect), f"replay {rep} differs from the eager call"


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("K", [5, 0])
def test_attn_graph_replay(case, K):
    _, make_graph, B, H, d, dtype = case
    g = make_graph()
    shape = (B, H, g.n, d)
    q, k, v = _inputs(shape, dtype, 500)
    out = torch.empty_like(v)
    ws = torch.empty(max(sah.workspace_size(g, B, H, d, d, dtype), 1), dtype=torch.uint8,
                     device=DEV)
    graph = _capture(lambda: sah.attn(q, k, v, g, K, 0.1, out=out, workspace=ws))
    _replay_matches_eager(graph, (q, k, v), out, shape, dtype,
                          lambda q2, k2, v2: sah.attn(q2, k2, v2, g, K, 0.1))


@pytest.mark.parametrize("case", [CASES[0], CASES[3]], ids=lambda c: c[0])
def test_attn_theta_graph_replay(case):
    _, make_graph, B, H, d, dtype = case
    g = make_graph()
    theta = [0.5, 0.25, 0.125, 0.125]
    shape = (B, H, g.n, d)
    q, k, v = _inputs(shape, dtype, 600)
    out = torch.empty_like(v)
    ws = torch.empty(max(sah.workspace_size(g, B, H, d, d, dtype), 1), dtype=torch.uint8,
                     device=DEV)
    graph = _capture(lambda: sah.attn_theta(q, k, v, g, theta, out=out, workspace=ws))
    _replay_matches_eager(graph, (q, k, v), out, shape, dtype,
                          lambda q2, k2, v2: sah.attn_theta(q2, k2, v2, g, theta))


@pytest.mark.parametrize("case", [CASES[0], CASES[3]], ids=lambda c: c[0])
def test_attn_backward_graph_replay(case):
    """The backward, once its first call has built the graph's column index
    (a one-time host step), also enqueues only kernel launches; its outputs
    are allocated inside the capture and rewritten by every replay."""
    _, make_graph, B, H, d, dtype = case
    g = make_graph()
    shape = (B, H, g.n, d)
    q, k, v = _inputs(shape, dtype, 700)
    dz = make_tensor(shape, 710, dtype).to(DEV)
    sah.attn_backward(q, k, v, dz, g, 3, 0.1)   # builds the column index
    torch.cuda.synchronize()
    got = {}

    def call():
        got["grads"] = sah.attn_backward(q, k, v, dz, g, 3, 0.1)

    graph = _capture(call)
    for rep in range(REPLAYS):
        new = _inputs(shape, dtype, 2000 + 10 * rep)
        for dst, src in zip((q, k, v), new):
            dst.copy_(src)
        for t in got["grads"]:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        expect = sah.attn_backward(*new, dz, g, 3, 0.1)
        torch.cuda.synchronize()
        for name, a, e in zip(("dq", "dk", "dv"), got["grads"], expect):
            assert torch.equal(a, e), f"replay {rep}: {name} differs from the eager call"
