"""GPU parity for the other static layouts: the BigBird block graph (eq. 13
of "1.2.1 Static sparsity", built by diffuser_build_block_graph; block 64
runs the block-tile kernels in bf16 with d = 64) and Longformer's dilated
window with globals (eqs. 11 and 12, diffuser_build_dilated_graph; generic
kernels). Graphs must match the oracle's bit for bit; weights and outputs
within parity_util's tolerances.
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


def _check_block_csr(orc, g, n, b, c, s, gb, ng, seed):
    rp, cols, _ = orc.block_graph(n, b, c, s, gb, ng, seed)
    for gr in range(ng):
        grp, gcols = g.copy_csr(gr)
        assert np.array_equal(grp, rp[gr]), f"row_ptr mismatch in graph {gr}"
        assert np.array_equal(gcols, cols[gr]), f"col_idx mismatch in graph {gr}"
    return rp, cols


BLOCK_SPECS = [
    # n, block, local, random, global, graphs, seed
    (48, 4, 3, 2, 1, 1, 0),          # the pages' twelve-block example
    (256, 64, 3, 1, 1, 2, 5),
    (512, 64, 3, 3, 2, 1, 7),
    (512, 64, 1, 0, 0, 1, 1),        # diagonal blocks only
    (384, 64, 5, 9, 1, 2, 3),        # random budget above the pool
    (128, 16, 9, 2, 0, 3, 9),        # local blocks beyond the sequence
    (1024, 8, 3, 4, 2, 2, 11),
]


@pytest.mark.parametrize("spec", BLOCK_SPECS, ids=lambda s: "n{}b{}c{}s{}g{}".format(*s[:5]))
def test_block_graph_csr_bitexact(orc, spec):
    n, b, c, s, gb, ng, seed = spec
    g = sah.build_block_graph(n, b, c, s, gb, ng, seed)
    _check_block_csr(orc, g, n, b, c, s, gb, ng, seed)


@pytest.mark.parametrize("n,r,dl,G", [(17, 2, 3, []), (200, 4, 7, [0, 99]), (64, 0, 5, [63]),
                                      (100, 60, 1, [3]), (1, 3, 2, [])])
def test_dilated_graph_csr_bitexact(orc, n, r, dl, G):
    g = sah.build_dilated_graph(n, r, dl, G)
    rp, cols = orc.dilated_graph(n, r, dl, G)
    grp, gcols = g.copy_csr(0)
    assert np.array_equal(grp, rp[0]) and np.array_equal(gcols, cols[0])


def test_layout_builders_invalid():
    bad_block = [
        (100, 64, 3, 1, 1),      # block does not divide n
        (128, 64, 2, 1, 1),      # even local count
        (128, 64, 3, -1, 1),     # negative random count
        (128, 64, 3, 1, 3),      # more global blocks than blocks
        (128, 0, 3, 1, 0),       # zero block
    ]
    for spec in bad_block:
        with pytest.raises(sah.DiffuserError) as ei:
            sah.build_block_graph(*spec)
        assert ei.value.status_name == "DIFFUSER_ERR_INVALID_ARG", spec
    for n, r, dl, G in [(10, -1, 1, []), (10, 1, 0, []), (10, 1, 1, [3, 3]), (10, 1, 1, [10])]:
        with pytest.raises(sah.DiffuserError):
            sah.build_dilated_graph(n, r, dl, G)


BLOCK_ATTN = [
    # n, block, local, random, global, graphs, B, H, d, dtype, K, alpha
    (256, 64, 3, 1, 1, 1, 2, 2, 64, "bf16", 5, 0.1),     # block-tile kernels
    (512, 64, 3, 3, 2, 2, 2, 3, 64, "bf16", 5, 0.1),     # block-tile kernels, per-batch graphs
    (512, 64, 5, 9, 1, 1, 1, 2, 64, "bf16", 3, 0.3),     # every block read (pool <= budget)
    (256, 64, 3, 1, 1, 1, 1, 2, 64, "f32", 5, 0.1),      # generic kernels on a block graph
    (96, 8, 3, 2, 1, 2, 2, 2, 32, "f32", 4, 0.2),        # small blocks: generic kernels
    (96, 8, 3, 2, 1, 1, 1, 2, 32, "bf16", 5, 0.1),
]


def _qkv(shape, seed, tdt):
    return (make_tensor(shape, seed, tdt), make_tensor(shape, seed + 1, tdt),
            make_tensor(shape, seed + 2, tdt))


@pytest.mark.parametrize("case", BLOCK_ATTN,
                         ids=lambda c: "n{}b{}s{}g{}B{}H{}d{}{}".format(c[0], c[1], c[3], c[4], c[6], c[7], c[8], c[9]))
def test_block_attn(orc, case):
    n, b, c, s, gb, ng, B, H, d, dt, K, alpha = case
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    g = sah.build_block_graph(n, b, c, s, gb, ng, 17)
    rp, cols = _check_block_csr(orc, g, n, b, c, s, gb, ng, 17)
    q, k, v = _qkv((B, H, n, d), 100 + n, tdt)
    z = _as64(sah.attn(q.to(DEV), k.to(DEV), v.to(DEV), g, K, alpha))
    for bb in range(B):
        gr = 0 if ng == 1 else bb
        for h in range(H):
            ref = orc.attn(_as64(q[bb, h]), _as64(k[bb, h]), _as64(v[bb, h]), rp[gr], cols[gr],
                           K, alpha, pu.oracle_threads())
            pu.assert_z_close(z[bb, h], ref, dt, f"b={bb} h={h}", K, alpha)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_block_scores_and_diffuse(orc, dt):
    """The normalised score pass alone (weights in CSR order) and one
    diffusion call on given weights, each against the oracle."""
    n, b, c, s, gb, B, H, d = 512, 64, 3, 2, 1, 2, 2, 64
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    g = sah.build_block_graph(n, b, c, s, gb, 1, 23)
    rp, cols = g.copy_csr(0)
    q, k, v = _qkv((B, H, n, d), 7, tdt)
    A = sah.scores_softmax(q.to(DEV), k.to(DEV), g)
    A_h = A.double().cpu().numpy()
    for bb in range(B):
        for h in range(H):
            off = g.a_offset(bb, h, H)
            got = A_h[off:off + g.slots[0]]
            ref = orc.scores_softmax(_as64(q[bb, h]), _as64(k[bb, h]), rp, cols)
            # the suite's bound for stored weights: bf16 rounding is at most
            # 2^-8 relative, plus an absolute 1e-6 for the normalisation by the
            # sum of rounded weights; fp32 1e-5 relative
            if dt == "f32":
                assert np.all(np.abs(got - ref) <= 1e-5 * ref + 1e-12), (bb, h)
            else:
                assert np.all(np.abs(got - ref) <= 2.0 ** -8 * ref + 1e-6), (bb, h)
            sums = np.add.reduceat(got, rp[:-1])
            assert np.all(np.abs(sums - 1.0) <= pu.rowsum_bound(dt)), (bb, h)
    z = _as64(sah.diffuse(A, v.to(DEV), g, 5, 0.1))
    for bb in range(B):
        for h in range(H):
            off = g.a_offset(bb, h, H)
            ref = orc.diffuse(A_h[off:off + g.slots[0]], _as64(v[bb, h]), rp, cols, 5, 0.1)
            pu.assert_z_close(z[bb, h], ref, dt, f"b={bb} h={h}")


def test_block_diffuse_default_workspace(orc):
    """Block graph with its global query blocks split over workgroups
    (n = 1024, 5 global blocks): diffuse and diffuse_theta with the
    workspace the query sizes, theta at K = 0 among them (one launch of the
    block step, whose partial sums need the workspace), and the C ABI's
    refusal of a NULL or short workspace for that launch."""
    import ctypes
    n, b, c, s, gb, B, H, d = 1024, 64, 3, 2, 5, 1, 2, 64
    g = sah.build_block_graph(n, b, c, s, gb, 1, 37)
    rp, cols = g.copy_csr(0)
    q, k, v = _qkv((B, H, n, d), 41, torch.bfloat16)
    A = sah.scores_softmax(q.to(DEV), k.to(DEV), g)
    vd = v.to(DEV)
    need0 = sah.diffuse_workspace_size(g, B, H, d, 0, torch.bfloat16)
    assert need0 > 0, "the split global blocks need partial sums"
    assert sah.diffuse_workspace_size(g, B, H, d, 5, torch.bfloat16) >= \
        need0 + v.numel() * v.element_size()
    A_h = A.double().cpu().numpy()
    z5 = _as64(sah.diffuse(A, vd, g, 5, 0.1))
    z0 = _as64(sah.diffuse_theta(A, vd, g, [1.0]))
    z2 = _as64(sah.diffuse_theta(A, vd, g, [0.5, 0.3, 0.2]))
    torch.cuda.synchronize()
    for h in range(H):
        off = g.a_offset(0, h, H)
        Ah = A_h[off:off + g.slots[0]]
        ref = orc.diffuse(Ah, _as64(v[0, h]), rp, cols, 5, 0.1)
        pu.assert_z_close(z5[0, h], ref, "bf16", f"K=5 h={h}")
        assert np.array_equal(z0[0, h], _as64(v[0, h])), f"theta [1] must give V, h={h}"
        ref2 = orc.diffuse_theta(Ah, _as64(v[0, h]), rp, cols, [0.5, 0.3, 0.2])
        pu.assert_z_close(z2[0, h], ref2, "bf16", f"theta K=2 h={h}", 2, 0.5)
    lib = sah.load_library()
    th = (ctypes.c_float * 1)(1.0)
    out = torch.empty_like(vd)
    ws = torch.empty(need0, dtype=torch.uint8, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for ptr, size in ((None, 0), (ws.data_ptr(), need0 - 256)):
        st = lib.diffuser_diffuse_theta(A.data_ptr(), vd.data_ptr(), 1, B, H, d, g.handle, 0, th,
                                        out.data_ptr(), ptr, size, stream)
        assert st == 1, f"workspace {size} bytes: status {st}"
    assert lib.diffuser_diffuse_theta(A.data_ptr(), vd.data_ptr(), 1, B, H, d, g.handle, 0, th,
                                      out.data_ptr(), ws.data_ptr(), need0, stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(out, vd)


def test_block_theta(orc):
    """General coefficients (eq. S.6) through the block-tile diffusion."""
    n, b, c, s, gb, B, H, d = 256, 64, 3, 1, 1, 1, 2, 64
    g = sah.build_block_graph(n, b, c, s, gb, 1, 4)
    rp, cols = g.copy_csr(0)
    q, k, v = _qkv((B, H, n, d), 31, torch.bfloat16)
    theta = [0.4, 0.3, 0.2, 0.1]
    z = _as64(sah.attn_theta(q.to(DEV), k.to(DEV), v.to(DEV), g, theta))
    for h in range(H):
        ref = orc.attn_theta(_as64(q[0, h]), _as64(k[0, h]), _as64(v[0, h]), rp, cols, theta)
        pu.assert_z_close(z[0, h], ref, "bf16", f"h={h}", len(theta) - 1, 0.1)


def test_block_attn_full_size(orc):
    """BigBird_D at the headline's shape (B 8, H 12, n 4096, d 64, bf16, K 5,
    alpha 0.1) with blocks of 64: 3 local, 3 random and 2 global blocks, a
    separate draw per batch element; sampled (b, h) pairs, every row."""
    n, b, c, s, gb, B, H, d = 4096, 64, 3, 3, 2, 8, 12, 64
    print(f"\n[parity] block graph n={n} block={b} local={c} random={s} global={gb} B={B} H={H}",
          flush=True)
    g = sah.build_block_graph(n, b, c, s, gb, B, 2024)
    q, k, v = _qkv((B, H, n, d), 900, torch.bfloat16)
    z = _as64(sah.attn(q.to(DEV), k.to(DEV), v.to(DEV), g, 5, 0.1))
    rp_all, cols_all, _ = orc.block_graph(n, b, c, s, gb, B, 2024)
    for bb, h in [(0, 0), (B - 1, H - 1), (3, 5)]:
        rp, cols = g.copy_csr(bb)
        assert np.array_equal(rp, rp_all[bb]) and np.array_equal(cols, cols_all[bb])
        ref = orc.attn(_as64(q[bb, h]), _as64(k[bb, h]), _as64(v[bb, h]), rp, cols, 5, 0.1,
                       pu.oracle_threads())
        pu.assert_z_close(z[bb, h], ref, "bf16", f"b={bb} h={h}")


@pytest.mark.parametrize("n", [512, 1024])
def test_block_far_maximum(orc, n):
    """Rows with a key scoring far above their own score: their shifted
    weights would pass 2^64, so the block-tile score kernel redoes them with
    the exact maximum (head 0); head 1 has ordinary inputs. At n = 1024 the
    global query block is split into parts."""
    b, c, s, gb = 64, 3, 2, 1
    g = sah.build_block_graph(n, b, c, s, gb, 1, 29)
    rp, cols = g.copy_csr(0)
    q, k, v = _qkv((1, 2, n, 64), 71, torch.bfloat16)
    far_key = n - 100
    q[0, 0] = 0
    q[0, 0, :, 0] = 16.0
    k[0, 0] = 0
    k[0, 0, far_key, 0] = 32.0        # score 64 for one key, 0 for every other one
    rows = np.repeat(np.arange(n), np.diff(rp))[cols == far_key]
    assert any(abs(int(i) - far_key) >= 2 * b for i in rows), "a non-local row must read it"
    A = _as64(sah.scores_softmax(q.to(DEV), k.to(DEV), g))
    z = _as64(sah.attn(q.to(DEV), k.to(DEV), v.to(DEV), g, 5, 0.1))
    for h in range(2):
        off = g.a_offset(0, h, 2)
        got = A[off:off + g.slots[0]]
        ref = orc.scores_softmax(_as64(q[0, h]), _as64(k[0, h]), rp, cols)
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * ref + 1e-6), h
        zref = orc.attn(_as64(q[0, h]), _as64(k[0, h]), _as64(v[0, h]), rp, cols, 5, 0.1)
        pu.assert_z_close(z[0, h], zref, "bf16", f"h={h}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_dilated_attn(orc, dt):
    n, r, dl, G, B, H, d = 300, 3, 4, [0, 150], 2, 2, 32
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    g = sah.build_dilated_graph(n, r, dl, G)
    rp, cols = orc.dilated_graph(n, r, dl, G)
    q, k, v = _qkv((B, H, n, d), 55, tdt)
    z = _as64(sah.attn(q.to(DEV), k.to(DEV), v.to(DEV), g, 5, 0.1))
    for bb in range(B):
        for h in range(H):
            ref = orc.attn(_as64(q[bb, h]), _as64(k[bb, h]), _as64(v[bb, h]), rp[0], cols[0], 5,
                           0.1)
            pu.assert_z_close(z[bb, h], ref, dt, f"b={bb} h={h}")


def test_block_backward(orc):
    """Gradients on a block graph (generic backward kernels) against the
    oracle's backward."""
    n, b, c, s, gb, B, H, d = 128, 16, 3, 1, 1, 1, 2, 32
    g = sah.build_block_graph(n, b, c, s, gb, 1, 8)
    rp, cols = g.copy_csr(0)
    q, k, v = _qkv((B, H, n, d), 61, torch.float32)
    dz = make_tensor((B, H, n, d), 64, torch.float32)
    dq, dk, dv = sah.attn_backward(q.to(DEV), k.to(DEV), v.to(DEV), dz.to(DEV), g, 3, 0.2)
    for h in range(H):
        rq, rk, rv = orc.attn_backward(_as64(q[0, h]), _as64(k[0, h]), _as64(v[0, h]),
                                       _as64(dz[0, h]), rp, cols, 3, 0.2)
        for got, ref, nm in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
            gg = _as64(got[0, h])
            scale = max(float(np.abs(ref).max()), 1e-6)
            assert float(np.abs(gg - ref).max()) <= 1e-4 * scale, (nm, h)
