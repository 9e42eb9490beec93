"""GPU parity of the CSR-order entry points (diffuser_scores_softmax_csr,
diffuser_diffuse_csr) against the oracle's CSR-ordered weights, with no
slot-layout permutation on the test side.

A_csr's (b, h) block is compared entry by entry with the oracle's edge
softmax over the same CSR; diffuse_csr is fed the oracle's weights (rounded
to the storage type), concatenated in CSR order, and its Z is compared with
the oracle's diffusion on the same rounded weights. Tolerances are those of
parity_util. One consistency check also ties the CSR output to the slot
layout's: the same bits, moved.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import parity_util as pu
import sparse_attention_hop_amd as sah
from workloads import make_tensor

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _as64(t):
    return t.double().cpu().numpy()


def _ragged_csr(n, seed):
    """A CSR of n rows with 1 .. n ascending columns per row, own index
    included (the import contract)."""
    rng = np.random.default_rng(seed)
    rows = []
    for i in range(n):
        k = int(rng.integers(0, n))
        s = set(rng.choice(n, size=k, replace=False).tolist()) | {i}
        rows.append(np.array(sorted(s), dtype=np.int32))
    rp = np.zeros(n + 1, np.int64)
    rp[1:] = np.cumsum([len(r) for r in rows])
    return rp, np.concatenate(rows)


def _built(n, r, G, R, ng, causal, seed):
    def make(orc):
        g = sah.build_graph(n, r, G, R, ng, causal, seed)
        rp, cols = orc.graph(n, r, G, R, ng, causal, seed)
        return g, [rp[gr] for gr in range(ng)], [cols[gr] for gr in range(ng)]
    return make


def _block(n, block, local, rnd, glob, ng, seed):
    def make(orc):
        g = sah.build_block_graph(n, block, local, rnd, glob, ng, seed)
        rp, cols, _ = orc.block_graph(n, block, local, rnd, glob, ng, seed)
        return g, [rp[gr] for gr in range(ng)], [cols[gr] for gr in range(ng)]
    return make


def _dilated(n, r, dil, G):
    def make(orc):
        g = sah.build_dilated_graph(n, r, dil, G)
        rp, cols = orc.dilated_graph(n, r, dil, G)
        return g, [rp[0]], [cols[0]]
    return make


def _imported(n, seeds):
    def make(orc):
        parts = [_ragged_csr(n, s) for s in seeds]
        rps = [p[0] for p in parts]
        cols = [p[1] for p in parts]
        g = sah.graph_from_csr(n, np.stack(rps), cols)
        return g, rps, cols
    return make


# id, graph maker, B, H, d, dtype
CASES = [
    ("octet_bf16_d64_2graphs", _built(1100, 50, [0, 1, 2, 700, 1099], 40, 2, False, 3), 2, 2, 64,
     torch.bfloat16),
    ("octet_bf16_d32_causal", _built(1024, 64, list(range(16)), 32, 1, True, 4), 1, 2, 32,
     torch.bfloat16),
    ("grouped_bf16_d64", _built(6000, 32, [0, 3000], 24, 1, False, 8), 1, 1, 64, torch.bfloat16),
    ("generic_f32_d16_3graphs", _built(300, 6, [0, 150], 9, 3, False, 5), 3, 2, 16,
     torch.float32),
    ("generic_f32_d128_causal", _built(257, 13, [3], 7, 1, True, 6), 1, 3, 128, torch.float32),
    ("block_bf16_d64", _block(1024, 64, 3, 2, 2, 1, 11), 1, 2, 64, torch.bfloat16),
    ("dilated_f32_d32", _dilated(333, 4, 3, [0, 100]), 2, 1, 32, torch.float32),
    ("imported_ragged_f32_2graphs", _imported(37, (1, 2)), 2, 2, 16, torch.float32),
    ("single_token_bf16", _built(1, 0, [], 0, 1, False, 0), 1, 1, 64, torch.bfloat16),
]


def _csr_block(nnz, ng, H, b, h):
    """Start of the (b, h) block of A_csr (nnz: edges per graph)."""
    if ng == 1:
        return (b * H + h) * nnz[0]
    return H * sum(nnz[:b]) + h * nnz[b]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_scores_softmax_csr_matches_oracle(orc, case):
    name, make, B, H, d, tdt = case
    print(f"\n[csr] {name}", flush=True)
    g, rps, cols = make(orc)
    ng = g.num_graphs
    for gr in range(ng):
        grp, gcols = g.copy_csr(gr)
        assert np.array_equal(grp, rps[gr]) and np.array_equal(gcols, cols[gr]), gr
    shape = (B, H, g.n, d)
    q = make_tensor(shape, 41, tdt)
    k = make_tensor(shape, 42, tdt)
    A_csr = sah.scores_softmax_csr(q.to(DEV), k.to(DEV), g)
    A_slots = sah.scores_softmax(q.to(DEV), k.to(DEV), g)
    torch.cuda.synchronize()
    assert A_csr.numel() == g.edges(B, H)
    A_h = _as64(A_csr)
    dt = pu.dtype_name(tdt)
    a_tol = 1e-5 if dt == "f32" else 2.0 ** -8 + 1e-5
    for b in range(B):
        gr = 0 if ng == 1 else b
        for h in range(H):
            off = _csr_block(g.nnz, ng, H, b, h)
            got = A_h[off:off + g.nnz[gr]]
            ref = orc.scores_softmax(_as64(q[b, h]), _as64(k[b, h]), rps[gr], cols[gr])
            assert np.all(np.abs(got - ref) <= a_tol * np.maximum(ref, 1e-30) + 1e-12), (b, h)
            sums = np.add.reduceat(got, rps[gr][:-1]) if g.n else got
            assert np.abs(sums - 1).max() <= pu.rowsum_bound(dt), (b, h)
    # the same bits as the slot layout's, each edge once
    s_h = A_slots.view(torch.int16 if tdt == torch.bfloat16 else torch.int32).cpu().numpy()
    c_h = A_csr.view(torch.int16 if tdt == torch.bfloat16 else torch.int32).cpu().numpy()
    assert np.array_equal(np.sort(s_h[s_h != 0]), np.sort(c_h[c_h != 0]))


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("K,alpha", [(0, 0.1), (3, 0.1), (5, 0.0)])
def test_diffuse_csr_matches_oracle(orc, case, K, alpha):
    name, make, B, H, d, tdt = case
    print(f"\n[csr] {name} K={K} alpha={alpha}", flush=True)
    g, rps, cols = make(orc)
    ng = g.num_graphs
    shape = (B, H, g.n, d)
    q = make_tensor(shape, 51, tdt)
    k = make_tensor(shape, 52, tdt)
    v = make_tensor(shape, 53, tdt)
    # the oracle's weights, rounded to the storage type, in CSR order
    blocks, refs = [], {}
    for b in range(B):
        gr = 0 if ng == 1 else b
        for h in range(H):
            a = orc.scores_softmax(_as64(q[b, h]), _as64(k[b, h]), rps[gr], cols[gr])
            a_t = torch.from_numpy(a).to(tdt)
            blocks.append(a_t)
            refs[(b, h)] = a_t.double().numpy()
    A_csr = torch.cat(blocks).to(DEV)
    assert A_csr.numel() == g.edges(B, H)
    z = sah.diffuse_csr(A_csr, v.to(DEV), g, K, alpha)
    torch.cuda.synchronize()
    z_h = _as64(z)
    dt = pu.dtype_name(tdt)
    for b in range(B):
        gr = 0 if ng == 1 else b
        for h in range(H):
            ref = orc.diffuse(refs[(b, h)], _as64(v[b, h]), rps[gr], cols[gr], K, alpha)
            pu.assert_z_close(z_h[b, h], ref, dt, f"{name} b={b} h={h}", K, alpha)


def test_csr_round_trip_through_diffuse():
    """diffuse_csr on scores_softmax_csr's output equals diffuse on the slot
    layout's weights bit for bit (same weights, same kernels)."""
    g = sah.build_graph(1100, 50, [0, 1, 2, 700, 1099], 40, 2, False, 3)
    shape = (2, 2, 1100, 64)
    q, k, v = (make_tensor(shape, s, torch.bfloat16).to(DEV) for s in (61, 62, 63))
    A_csr = sah.scores_softmax_csr(q, k, g)
    A = sah.scores_softmax(q, k, g)
    z1 = sah.diffuse_csr(A_csr, v, g, 4, 0.1)
    z2 = sah.diffuse(A, v, g, 4, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(z1, z2)


def test_csr_invalid_arguments():
    g = sah.build_graph(200, 4, [0], 3, 1, False, 1)
    lib = sah.load_library()
    B, H, d = 1, 1, 64
    v = torch.zeros(B, H, 200, d, dtype=torch.float32, device=DEV)
    a = torch.zeros(g.edges(B, H), dtype=torch.float32, device=DEV)
    z = torch.empty_like(v)
    need = sah.csr_workspace_size(g, B, H, d, 3, torch.float32)
    assert need >= g.a_numel(B, H) * 4
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    f32 = 0
    # workspace too small
    assert lib.diffuser_diffuse_csr(a.data_ptr(), v.data_ptr(), f32, B, H, d, g.handle, 3, 0.1,
                                    z.data_ptr(), ws.data_ptr(), need - 1, None) == 1
    # A_csr inside the workspace
    assert lib.diffuser_diffuse_csr(ws.data_ptr(), v.data_ptr(), f32, B, H, d, g.handle, 3, 0.1,
                                    z.data_ptr(), ws.data_ptr(), need, None) == 1
    # alpha out of range
    assert lib.diffuser_diffuse_csr(a.data_ptr(), v.data_ptr(), f32, B, H, d, g.handle, 3, 1.5,
                                    z.data_ptr(), ws.data_ptr(), need, None) == 1
    # scores: workspace too small, and A_csr overlapping the workspace
    need_s = g.a_numel(B, H) * 4
    assert lib.diffuser_scores_softmax_csr(v.data_ptr(), v.data_ptr(), f32, B, H, d, g.handle,
                                           a.data_ptr(), ws.data_ptr(), need_s // 2, None) == 1
    assert lib.diffuser_scores_softmax_csr(v.data_ptr(), v.data_ptr(), f32, B, H, d, g.handle,
                                           ws.data_ptr(), ws.data_ptr(), need, None) == 1
    torch.cuda.synchronize()
