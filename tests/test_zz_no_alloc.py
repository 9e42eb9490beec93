"""diffuser_diffuse_noalloc, the entry point that allocates nothing, against
diffuser_diffuse on the same inputs: two calls in a row (the second on a
smaller input, so the library's scratch array holds the first call's data
when the second starts), on a token graph (resident-slice step), a block
graph with split global blocks (whose partial sums live in the scratch)
and the headline shape (Z buffer of 48 MiB). The kernels are the same, so
the outputs must be equal bit for bit. Requests beyond the array's 64 MiB
are refused before any launch."""
from __future__ import annotations

import ctypes

import pytest
import torch

import sparse_attention_hop_amd as sah
from workloads import make_tensor

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _pair(g, B, H, d, K, alpha, seed):
    q = make_tensor((B, H, g.n, d), seed, torch.bfloat16).to(DEV)
    k = make_tensor((B, H, g.n, d), seed + 1, torch.bfloat16).to(DEV)
    v = make_tensor((B, H, g.n, d), seed + 2, torch.bfloat16).to(DEV)
    A = sah.scores_softmax(q, k, g)
    ws = torch.empty(max(sah.diffuse_workspace_size(g, B, H, d, K, v.dtype), 1),
                     dtype=torch.uint8, device=DEV)
    ref = sah.diffuse(A, v, g, K, alpha, workspace=ws)
    out = torch.full_like(v, float("nan"))
    got = sah.diffuse_noalloc(A, v, g, K, alpha, out)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), f"n={g.n} B={B} H={H} d={d} K={K}: differs from diffuser_diffuse"


def test_noalloc_matches_diffuse_token_graphs():
    print("\n[noalloc] token graphs: n=1100 d=64 K=5, then n=600 d=32 K=3", flush=True)
    g1 = sah.build_graph(1100, 50, [0, 1, 2, 700, 1099], 40, 2, False, 3)
    _pair(g1, 2, 3, 64, 5, 0.1, 10)
    g2 = sah.build_graph(600, 16, [0, 300], 12, 1, True, 7)
    _pair(g2, 1, 2, 32, 3, 0.3, 20)


def test_noalloc_matches_diffuse_block_graph():
    print("\n[noalloc] block graph n=1024, 5 global blocks, K=4, then n=512 K=2", flush=True)
    g1 = sah.build_block_graph(1024, 64, 3, 2, 5, 1, 37)
    _pair(g1, 1, 2, 64, 4, 0.1, 30)
    g2 = sah.build_block_graph(512, 64, 3, 1, 1, 1, 5)
    _pair(g2, 1, 2, 64, 2, 0.2, 40)


def test_noalloc_headline_then_small():
    print("\n[noalloc] headline shape B=8 H=12 n=4096 d=64 K=5, then n=300 K=2", flush=True)
    G = list(range(64))
    g1 = sah.build_graph(4096, 64, G, 64, 8, False, 1003)
    _pair(g1, 8, 12, 64, 5, 0.1, 50)
    g2 = sah.build_graph(300, 6, [0, 150], 9, 1, False, 31)
    _pair(g2, 1, 1, 64, 2, 0.1, 60)


def test_noalloc_no_scratch_and_refusals():
    """K = 0 and 1 need no scratch; a request beyond 64 MiB is refused."""
    g = sah.build_graph(300, 6, [0, 150], 9, 1, False, 31)
    for K in (0, 1):
        _pair(g, 2, 2, 64, K, 0.1, 70 + K)
    lib = sah.load_library()
    small = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # B * H * n * d * 2 bytes = 4000 * 300 * 64 * 2 > 64 MiB (one graph shared)
    st = lib.diffuser_diffuse_noalloc(small.data_ptr(), small.data_ptr(), 1, 1000, 4, 64,
                                      g.handle, 5, ctypes.c_float(0.1), small.data_ptr(), stream)
    msg = lib.diffuser_last_error().decode()
    assert st == 1 and "bytes of scratch" in msg, (st, msg)
