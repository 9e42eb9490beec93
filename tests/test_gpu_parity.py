"""GPU parity: the HIP path through the C ABI against the CPU oracle.

CSR graphs must match bit for bit; edge weights and outputs must agree
within the tolerances of parity_util. Full-size workloads are compared on
sampled (batch, head) pairs, every row of each; small randomized shapes are
compared everywhere.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle_pins
import parity_util as pu
import sparse_attention_hop_amd as sah
from workloads import WORKLOADS, make_qkv, make_tensor, sweep_variants

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _gpu_graph(n, r, G, R, ng, causal, seed):
    return sah.build_graph(n, r, G, R, ng, causal, seed)


def _check_csr(orc, g, n, r, G, R, ng, causal, seed):
    rp, cols = orc.graph(n, r, G, R, ng, causal, seed)
    for gr in range(ng):
        grp, gcols = g.copy_csr(gr)
        assert np.array_equal(grp, rp[gr]), f"row_ptr mismatch in graph {gr}"
        assert np.array_equal(gcols, cols[gr]), f"col_idx mismatch in graph {gr}"
        sr, sc = g.copy_slots(gr)
        pu.slot_permutation(sr, sc, rp[gr], cols[gr])
        assert len(sc) % 8 == 0, "segments and groups are multiples of 8 slots"
    return rp, cols


def _a_csr(g, A_h, b, h, H, gr, rp, cols):
    """The (b, h) block of A (slot layout) in ascending-CSR order; padding
    slots must hold exactly 0."""
    sr, sc = g.copy_slots(gr)
    perm, pad = pu.slot_permutation(sr, sc, rp[gr], cols[gr])
    off = g.a_offset(b, h, H)
    blk = A_h[off:off + g.slots[gr]]
    assert np.all(blk[pad] == 0), "padding slots must hold 0"
    return blk[perm]


def _as64(t):
    return t.double().cpu().numpy()


# ---------------------------------------------------------------------------
# Graph builder: bit-exact CSR
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(WORKLOADS))
def test_csr_bitexact_workloads(orc, name):
    w = WORKLOADS[name]
    g = _gpu_graph(w.n, w.radius, w.global_idx, w.num_random, w.num_graphs, w.causal,
                   w.graph_seed)
    _check_csr(orc, g, w.n, w.radius, w.global_idx, w.num_random, w.num_graphs, w.causal,
               w.graph_seed)


@pytest.mark.parametrize("R", [0, 32, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_csr_bitexact_sweep(orc, R, causal):
    w = WORKLOADS["sweep8192_f32"]
    g = _gpu_graph(w.n, w.radius, w.global_idx, R, 1, causal, w.graph_seed)
    _check_csr(orc, g, w.n, w.radius, w.global_idx, R, 1, causal, w.graph_seed)


def _random_specs(count, seed):
    rng = np.random.default_rng(seed)
    specs = []
    for _ in range(count):
        n = int(rng.integers(1, 301))
        r = int(rng.choice([0, 1, 2, 5, 17, n]))
        g = int(rng.integers(0, min(n, 6) + 1))
        G = sorted(rng.choice(n, size=g, replace=False).tolist()) if g else []
        R = int(rng.choice([0, 1, 3, 8, 40, n]))
        ng = int(rng.choice([1, 2, 3]))
        causal = bool(rng.integers(0, 2))
        specs.append((n, r, G, R, ng, causal, int(rng.integers(0, 2 ** 63))))
    return specs


@pytest.mark.parametrize("spec", _random_specs(40, 1), ids=lambda s: f"n{s[0]}r{s[1]}g{len(s[2])}R{s[3]}")
def test_csr_bitexact_random(orc, spec):
    g = _gpu_graph(*spec)
    _check_csr(orc, g, *spec)


def test_csr_edge_cases(orc):
    for spec in [(1, 0, [], 0, 1, False, 0), (1, 3, [0], 5, 2, True, 1),
                 (7, 0, [], 0, 1, False, 2), (9, 0, list(range(9)), 3, 1, False, 3),
                 (64, 100, [], 0, 1, True, 4), (50, 2, [0, 49], 1000, 1, False, 5),
                 (2000, 3, [1000], 1024, 1, False, 6)]:
        g = _gpu_graph(*spec)
        _check_csr(orc, g, *spec)


# ---------------------------------------------------------------------------
# Whole path at the workloads' full sizes, sampled (b, h) pairs
# ---------------------------------------------------------------------------

def _samples(B, H):
    pairs = {(0, 0), (B - 1, H - 1), (B // 2, H // 3)}
    return sorted(pairs)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_attn_full_size(orc, name):
    w = WORKLOADS[name]
    print(f"\n[parity] {w.describe()}", flush=True)
    g = _gpu_graph(w.n, w.radius, w.global_idx, w.num_random, w.num_graphs, w.causal,
                   w.graph_seed)
    rp, cols = _check_csr(orc, g, w.n, w.radius, w.global_idx, w.num_random, w.num_graphs,
                          w.causal, w.graph_seed)
    q, k, v = make_qkv(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    A = sah.scores_softmax(qd, kd, g)
    z = sah.attn(qd, kd, vd, g, w.K, w.alpha)
    torch.cuda.synchronize()
    A_h = _as64(A)
    threads = pu.oracle_threads()
    pairs = _samples(w.B, w.H)
    for b, h in pairs:
        gr = 0 if w.num_graphs == 1 else b
        A_ref = orc.scores_softmax(_as64(q[b, h]), _as64(k[b, h]), rp[gr], cols[gr], threads)
        A_got = _a_csr(g, A_h, b, h, w.H, gr, rp, cols)
        bound = pu.rowsum_bound(w.dtype)
        sums = np.add.reduceat(A_got, rp[gr][:-1])
        assert np.abs(sums - 1).max() <= bound, (b, h, np.abs(sums - 1).max())
        a_tol = 1e-5 if w.dtype == "f32" else 2.0 ** -8 + 1e-5
        assert np.all(np.abs(A_got - A_ref) <= a_tol * np.maximum(A_ref, 1e-30) + 1e-12), (b, h)
        z_ref = orc.diffuse(A_ref, _as64(v[b, h]), rp[gr], cols[gr], w.K, w.alpha, threads)
        e = pu.assert_z_close(_as64(z[b, h]), z_ref, w.dtype, f"{name} b={b} h={h}")
        print(f"[parity] {name} b={b} h={h} err={e:.3e} x tol", flush=True)


@pytest.mark.parametrize("R", [0, 32, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_sweep_full_size(orc, R, causal):
    base = WORKLOADS["sweep8192_f32"]
    variants = [w for w in sweep_variants() if w.num_random == R and w.causal == causal]
    g = _gpu_graph(base.n, base.radius, base.global_idx, R, 1, causal, base.graph_seed)
    rp, cols = _check_csr(orc, g, base.n, base.radius, base.global_idx, R, 1, causal,
                          base.graph_seed)
    q, k, v = make_qkv(base)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    threads = pu.oracle_threads()
    pairs = _samples(base.B, base.H)
    # A on every sampled pair, element by element, and its row sums.
    A = sah.scores_softmax(qd, kd, g)
    A_h = _as64(A)
    A_refs = {}
    for b, h in pairs:
        A_ref = orc.scores_softmax(_as64(q[b, h]), _as64(k[b, h]), rp[0], cols[0], threads)
        A_got = _a_csr(g, A_h, b, h, base.H, 0, rp, cols)
        assert np.all(np.abs(A_got - A_ref) <= 1e-5 * A_ref + 1e-12), (b, h)
        sums = np.add.reduceat(A_got, rp[0][:-1])
        assert np.abs(sums - 1).max() <= pu.rowsum_bound("f32"), (b, h)
        A_refs[(b, h)] = A_ref
    worst = 0.0
    for w in variants:
        z = _as64(sah.attn(qd, kd, vd, g, w.K, w.alpha))
        for b, h in pairs:
            z_ref = orc.diffuse(A_refs[(b, h)], _as64(v[b, h]), rp[0], cols[0], w.K, w.alpha,
                                threads)
            worst = max(worst, pu.assert_z_close(z[b, h], z_ref, "f32", f"{w.name} b={b} h={h}"))
    print(f"\n[parity] sweep R={R} causal={causal}: {len(variants)} variants x "
          f"{len(pairs)} pairs, worst {worst:.3e} x tol", flush=True)


# ---------------------------------------------------------------------------
# Small randomized shapes, compared on every (b, h)
# ---------------------------------------------------------------------------

def _small_cases(count, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for c in range(count):
        n = int(rng.integers(1, 301))
        r = int(rng.choice([0, 1, 4, 13, 40, n]))
        g = int(rng.integers(0, min(n, 5) + 1))
        G = sorted(rng.choice(n, size=g, replace=False).tolist()) if g else []
        R = int(rng.choice([0, 2, 7, 33]))
        B = int(rng.integers(1, 4))
        H = int(rng.integers(1, 4))
        ng = int(rng.choice([1, B]))
        causal = bool(rng.integers(0, 2))
        d = int(rng.choice([16, 32, 64, 128]))
        dtype = "f32" if rng.integers(0, 2) else "bf16"
        K = int(rng.choice([0, 1, 2, 5, 10]))
        alpha = float(rng.choice([0.0, 0.05, 0.1, 0.3, 1.0]))
        cases.append(dict(n=n, r=r, G=G, R=R, B=B, H=H, ng=ng, causal=causal, d=d,
                          dtype=dtype, K=K, alpha=alpha, seed=100 + c))
    return cases


@pytest.mark.parametrize("case", _small_cases(48, 7),
                         ids=lambda c: f"n{c['n']}d{c['d']}{c['dtype']}K{c['K']}")
def test_attn_small_random(orc, case):
    c = case
    tdt = torch.float32 if c["dtype"] == "f32" else torch.bfloat16
    g = _gpu_graph(c["n"], c["r"], c["G"], c["R"], c["ng"], c["causal"], c["seed"])
    rp, cols = _check_csr(orc, g, c["n"], c["r"], c["G"], c["R"], c["ng"], c["causal"],
                          c["seed"])
    shape = (c["B"], c["H"], c["n"], c["d"])
    q = make_tensor(shape, c["seed"], tdt)
    k = make_tensor(shape, c["seed"] + 1, tdt)
    v = make_tensor(shape, c["seed"] + 2, tdt)
    z = sah.attn(q.to(DEV), k.to(DEV), v.to(DEV), g, c["K"], c["alpha"])
    z_h = _as64(z)
    for b in range(c["B"]):
        gr = 0 if c["ng"] == 1 else b
        for h in range(c["H"]):
            ref = orc.attn(_as64(q[b, h]), _as64(k[b, h]), _as64(v[b, h]), rp[gr], cols[gr],
                           c["K"], c["alpha"])
            pu.assert_z_close(z_h[b, h], ref, c["dtype"], f"b={b} h={h}", c["K"], c["alpha"])


# ---------------------------------------------------------------------------
# The pages' worked examples through the C ABI
# ---------------------------------------------------------------------------

def test_softmax_8pos_gpu():
    """n=8, radius 1, query position 4 (index 3): scores (0, ln 2, 0) give
    weights (1/4, 1/2, 1/4) and, with alpha=0, K=1, output (1, 1.5)."""
    gold = oracle_pins.golden_dict("softmax_8pos.txt")
    g = sah.build_graph(8, 1, [], 0)
    d = 32
    q = torch.zeros(1, 1, 8, d)
    k = torch.zeros(1, 1, 8, d)
    q[0, 0, 3, 0] = math.sqrt(d)
    k[0, 0, 3, 0] = float(gold["scores"][1])
    v = torch.zeros(1, 1, 8, d)
    v[0, 0, 2, :2] = torch.tensor([float(x) for x in gold["v3"]])
    v[0, 0, 3, :2] = torch.tensor([float(x) for x in gold["v4"]])
    v[0, 0, 4, :2] = torch.tensor([float(x) for x in gold["v5"]])
    A = sah.scores_softmax(q.to(DEV), k.to(DEV), g).cpu().numpy()
    rp, cols = g.copy_csr(0)
    A_csr = _a_csr(g, A, 0, 0, 1, 0, [rp], [cols])
    want = np.array([float(x) for x in gold["weights"]])
    assert np.allclose(A_csr[rp[3]:rp[4]], want, rtol=0, atol=1e-6)
    z = sah.attn(q.to(DEV), k.to(DEV), v.to(DEV), g, 1, 0.0).cpu().numpy()
    assert np.allclose(z[0, 0, 3, :2], [float(x) for x in gold["o4"]], rtol=0, atol=1e-6)
    assert np.all(z[0, 0, 3, 2:] == 0)


def test_three_token_gpu():
    """Imported CSR {0:[0,1], 1:[1,2], 2:[2]}, alpha=0.1, K=2, V=[I|0]: the
    first row of Z is (0.3475, 0.45, 0.2025)."""
    gold = oracle_pins.golden_dict("diffusion_3token.txt")
    rp = np.array([[0, 2, 4, 5]], dtype=np.int64)
    cols = np.array([0, 1, 1, 2, 2], dtype=np.int32)
    g = sah.graph_from_csr(3, rp, cols)
    A = torch.tensor([0.5, 0.5, 0.5, 0.5, 1.0], dtype=torch.float32, device=DEV)
    v = torch.zeros(1, 1, 3, 32)
    v[0, 0, :, :3] = torch.eye(3)
    z = sah.diffuse(A, v.to(DEV), g, int(gold["K"][0]), float(gold["alpha"][0])).cpu().numpy()
    want = [float(x) for x in gold["Z2_row0_coeffs"]]
    assert np.allclose(z[0, 0, 0, :3], want, rtol=0, atol=1e-6), z[0, 0, 0, :3]


# ---------------------------------------------------------------------------
# Properties on the GPU
# ---------------------------------------------------------------------------

def _setup(n=300, r=6, G=(0, 150), R=9, causal=False, dtype=torch.float32, B=2, H=3, d=64):
    g = sah.build_graph(n, r, list(G), R, 1, causal, 77)
    shape = (B, H, n, d)
    q, k, v = (make_tensor(shape, 5 + i, dtype).to(DEV) for i in range(3))
    return g, q, k, v


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_identity_cases_bitwise(dtype):
    g, q, k, v = _setup(dtype=dtype)
    assert torch.equal(sah.attn(q, k, v, g, 0, 0.1), v)
    assert torch.equal(sah.attn(q, k, v, g, 5, 1.0), v)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_determinism(dtype):
    g, q, k, v = _setup(dtype=dtype)
    z1 = sah.attn(q, k, v, g, 5, 0.1)
    z2 = sah.attn(q, k, v, g, 5, 0.1)
    assert torch.equal(z1, z2)


def test_causality_gpu():
    g, q, k, v = _setup(causal=True)
    z0 = sah.attn(q, k, v, g, 5, 0.1)
    for p in (0, 77, 299):
        v2 = v.clone()
        v2[:, :, p] += 1.0
        z1 = sah.attn(q, k, v2, g, 5, 0.1)
        assert torch.equal(z0[:, :, :p], z1[:, :, :p]), p
        assert not torch.equal(z0[:, :, p], z1[:, :, p])


def test_reach_gpu():
    n, r, K, p = 200, 4, 3, 100
    g, q, k, v = _setup(n=n, r=r, G=(), R=0)
    z0 = sah.attn(q, k, v, g, K, 0.1)
    v2 = v.clone()
    v2[:, :, p] += 1.0
    z1 = sah.attn(q, k, v2, g, K, 0.1)
    changed = (z0 != z1).any(dim=-1).any(dim=0).any(dim=0).cpu().numpy()
    assert np.array_equal(changed, np.abs(np.arange(n) - p) <= K * r)


def test_constant_v_fixed_point_gpu():
    g, q, k, v = _setup()
    row = make_tensor((1, 1, 1, 64), 9).to(DEV)
    vc = row.expand_as(v).contiguous()
    z = sah.attn(q, k, vc, g, 7, 0.1)
    assert torch.allclose(z, vc, rtol=1e-5, atol=1e-6)


def test_rowsums_bf16():
    g, q, k, v = _setup(dtype=torch.bfloat16)
    A = sah.scores_softmax(q, k, g).double().cpu().numpy()
    sr, _ = g.copy_slots(0)
    ns = g.slots[0]
    valid = sr >= 0
    for bh in range(6):
        sums = np.bincount(sr[valid], weights=A[bh * ns:(bh + 1) * ns][valid], minlength=g.n)
        assert np.abs(sums - 1).max() <= pu.ROWSUM_BF16


# ---------------------------------------------------------------------------
# Boundary behaviour
# ---------------------------------------------------------------------------

def test_invalid_arguments_gpu():
    g, q, k, v = _setup()
    with pytest.raises(sah.DiffuserError) as ei:
        sah.attn(q, k, v, g, -1, 0.1)
    assert ei.value.status == 1
    with pytest.raises(sah.DiffuserError):
        sah.attn(q, k, v, g, 5, 1.5)
    with pytest.raises(sah.DiffuserError) as ei:
        sah.attn(q[..., :48].contiguous(), k[..., :48].contiguous(), v[..., :48].contiguous(),
                 g, 5, 0.1)
    assert ei.value.status == 2
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(sah.DiffuserError):
        sah.attn(q, k, v, g, 5, 0.1, workspace=ws)
    with pytest.raises(sah.DiffuserError):
        sah.attn(q, k, v, g, 5, 0.1, out=v)          # Z aliases V
    with pytest.raises(sah.DiffuserError):
        sah.build_graph(10, 1, [4, 2], 0)
    with pytest.raises(sah.DiffuserError):
        sah.graph_from_csr(3, np.array([[0, 1, 2, 3]]), np.array([1, 0, 2], dtype=np.int32))
    gB = sah.build_graph(300, 6, [0], 9, 3, False, 1)
    with pytest.raises(sah.DiffuserError):
        sah.attn(q, k, v, gB, 5, 0.1)                # num_graphs not in {1, B}


# ---------------------------------------------------------------------------
# LDS-streamed MFMA kernels (built graphs, bf16, d = 64 or 32): shapes that cross
# chunk and tile boundaries, several global-row workgroups, causal rows,
# empty random sets, windows wider than the sequence.
# ---------------------------------------------------------------------------

FAST_CASES = [
    # n, r, G, R, num_graphs(B), causal, B, H
    (300, 6, [0, 150], 9, 1, False, 2, 3),
    (700, 20, list(range(0, 700, 7))[:70], 12, 2, False, 2, 2),
    (513, 64, list(range(64)), 64, 1, False, 1, 2),
    (1000, 3, [5, 999], 0, 1, True, 1, 3),
    (257, 300, [], 5, 1, False, 1, 1),
    (64, 1, [], 3, 1, True, 2, 1),
    (1100, 50, [0, 1, 2, 700, 1099], 40, 3, True, 3, 1),
    (33, 2, [32], 40, 1, False, 1, 1),
    # B * H a multiple of 8: the score kernel numbers its work items per XCD
    # by (b, h); every pair is compared
    (600, 16, [0, 300], 12, 1, False, 2, 4),
    (520, 24, [0, 1, 519], 10, 4, False, 4, 4),
    # near the whole-sequence resident step's limits: one 32-channel plane
    # pair only just fits (n = 2300, no globals), a single 16-channel plane
    # up to the longest octet-layout sequence (4576), causal rows
    (3000, 40, [0, 1500, 2999], 30, 1, False, 1, 2),
    (4576, 64, list(range(64)), 64, 2, True, 2, 1),
    (2300, 8, [], 20, 1, False, 1, 3),
    (4100, 100, list(range(0, 4100, 85)), 48, 1, False, 1, 2),
]


@pytest.mark.parametrize("case", FAST_CASES, ids=lambda c: f"n{c[0]}r{c[1]}g{len(c[2])}R{c[3]}c{int(c[5])}")
@pytest.mark.parametrize("K,alpha", [(5, 0.1), (2, 0.0), (1, 0.3)])
@pytest.mark.parametrize("d", [64, 32])
def test_fast_diffusion_shapes(orc, case, K, alpha, d):
    n, r, G, R, ngr, causal, B, H = case
    ng = ngr if ngr in (1, B) else B
    g = _gpu_graph(n, r, G, R, ng, causal, 31)
    rp, cols = _check_csr(orc, g, n, r, G, R, ng, causal, 31)
    shape = (B, H, n, d)
    q = make_tensor(shape, 71, torch.bfloat16)
    k = make_tensor(shape, 72, torch.bfloat16)
    v = make_tensor(shape, 73, torch.bfloat16)
    z = sah.attn(q.to(DEV), k.to(DEV), v.to(DEV), g, K, alpha)
    # the stage entry (no row rescale) must match the oracle on the given A
    A = sah.scores_softmax(q.to(DEV), k.to(DEV), g)
    zs = sah.diffuse(A, v.to(DEV), g, K, alpha)
    z_h, zs_h, A_h = _as64(z), _as64(zs), _as64(A)
    for b in range(B):
        gr = 0 if ng == 1 else b
        for h in range(H):
            ref = orc.attn(_as64(q[b, h]), _as64(k[b, h]), _as64(v[b, h]), rp[gr], cols[gr], K,
                           alpha)
            pu.assert_z_close(z_h[b, h], ref, "bf16", f"attn b={b} h={h}", K, alpha)
            A_csr = _a_csr(g, A_h, b, h, H, gr, rp, cols)
            A_ref = orc.scores_softmax(_as64(q[b, h]), _as64(k[b, h]), rp[gr], cols[gr])
            assert np.all(np.abs(A_csr - A_ref) <= 2.0 ** -8 * A_ref + 1e-6), (b, h)
            ref_s = orc.diffuse(A_csr, _as64(v[b, h]), rp[gr], cols[gr], K, alpha)
            # same stored A on both sides: only the Z_k roundings differ
            pu.assert_z_close(zs_h[b, h], ref_s, "bf16", f"diffuse b={b} h={h}", K, alpha)


DRIFT_CASES = [
    # id, graph builder, B, H, d
    ("octet_d64", lambda: sah.build_graph(1100, 50, [0, 1, 2, 700, 1099], 40, 2, False, 3), 2, 2, 64),
    ("octet_d32_causal", lambda: sah.build_graph(1024, 64, list(range(16)), 32, 1, True, 4), 1, 2, 32),
    ("grouped_d64", lambda: sah.build_graph(6000, 32, [0, 3000], 24, 1, False, 8), 1, 1, 64),
    ("block_d64", lambda: sah.build_block_graph(1024, 64, 3, 2, 2, 1, 11), 1, 2, 64),
    ("generic_d128", lambda: sah.build_graph(700, 20, [3, 400], 16, 1, False, 5), 1, 2, 128),
]


@pytest.mark.parametrize("case", DRIFT_CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("K,alpha", [(10, 0.0), (10, 0.05)])
def test_bf16_long_diffusion_plain_bound(orc, case, K, alpha):
    """Ten steps with no or little restart, where bf16 rounding has the most
    steps to build up: Z within the plain 2e-2 bound of K = 5, alpha = 0.1
    (the row rescale keeps every step's matrix row-stochastic, so the
    error does not grow with K). Prints the worst error in units of it."""
    _, make_graph, B, H, d = case
    g = make_graph()
    rps, colss = [], []
    for gr in range(len(g.nnz)):
        rp, cols = g.copy_csr(gr)
        rps.append(rp)
        colss.append(cols)
    shape = (B, H, g.n, d)
    q = make_tensor(shape, 91, torch.bfloat16)
    k = make_tensor(shape, 92, torch.bfloat16)
    v = make_tensor(shape, 93, torch.bfloat16)
    z = _as64(sah.attn(q.to(DEV), k.to(DEV), v.to(DEV), g, K, alpha))
    worst = 0.0
    for b in range(B):
        gr = 0 if len(rps) == 1 else b
        for h in range(H):
            ref = orc.attn(_as64(q[b, h]), _as64(k[b, h]), _as64(v[b, h]), rps[gr], colss[gr], K,
                           alpha, pu.oracle_threads())
            worst = max(worst, pu.z_error(z[b, h], ref, "bf16", 5, 0.1))
    print(f"\n[drift] {case[0]} K={K} alpha={alpha}: worst error {worst:.3f} x 2e-2", flush=True)
    assert worst <= 1.0, f"error {worst:.3f} x the plain 2e-2 bound"


@pytest.mark.parametrize("n", [1 << 16, (1 << 16) + 1])
def test_longest_scheduled_sequence(orc, n):
    """The longest sequence that gets the random schedule (2^16 tokens, the
    LDS-streamed kernels) and one token more (row-segment random slots, the
    generic kernels): graph bit-exact, weights and Z against the oracle."""
    r, G, R = 32, [0, n // 2, n - 1], 16
    print(f"\n[parity] n={n} r={r} g={len(G)} R={R}", flush=True)
    g = _gpu_graph(n, r, G, R, 1, False, 57)
    rp, cols = _check_csr(orc, g, n, r, G, R, 1, False, 57)
    shape = (1, 1, n, 64)
    q = make_tensor(shape, 81, torch.bfloat16)
    k = make_tensor(shape, 82, torch.bfloat16)
    v = make_tensor(shape, 83, torch.bfloat16)
    z = _as64(sah.attn(q.to(DEV), k.to(DEV), v.to(DEV), g, 3, 0.1))
    A = _as64(sah.scores_softmax(q.to(DEV), k.to(DEV), g))
    A_csr = _a_csr(g, A, 0, 0, 1, 0, rp, cols)
    A_ref = orc.scores_softmax(_as64(q[0, 0]), _as64(k[0, 0]), rp[0], cols[0])
    assert np.all(np.abs(A_csr - A_ref) <= 2.0 ** -8 * A_ref + 1e-6)
    ref = orc.attn(_as64(q[0, 0]), _as64(k[0, 0]), _as64(v[0, 0]), rp[0], cols[0], 3, 0.1,
                   pu.oracle_threads())
    pu.assert_z_close(z[0, 0], ref, "bf16", f"n={n}", 3, 0.1)


@pytest.mark.parametrize("case", [FAST_CASES[1], FAST_CASES[6]],
                         ids=lambda c: f"n{c[0]}r{c[1]}g{len(c[2])}R{c[3]}c{int(c[5])}")
def test_fast_paths_deterministic(case):
    """Repeated calls give bitwise-equal A and Z (no ordering or LDS race
    shows through)."""
    n, r, G, R, ngr, causal, B, H = case
    ng = ngr if ngr in (1, B) else B
    g = _gpu_graph(n, r, G, R, ng, causal, 31)
    shape = (B, H, n, 64)
    q, k, v = (make_tensor(shape, 81 + i, torch.bfloat16).to(DEV) for i in range(3))
    A0 = sah.scores_softmax(q, k, g)
    z0 = sah.attn(q, k, v, g, 5, 0.1)
    for _ in range(3):
        assert torch.equal(sah.scores_softmax(q, k, g), A0)
        assert torch.equal(sah.attn(q, k, v, g, 5, 0.1), z0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 32])
def test_fast_scores_far_random_maximum(orc, causal, d):
    """Rows whose maximum score is a random (or, for a global row, a
    late-chunk) edge far above the window: the shifted weights would pass
    2^64, so the kernel redoes those rows with their exact maximum. Head 0
    has that structure, head 1 ordinary inputs."""
    n, r, G, R = 1100, 20, [0, 1, 700], 40
    g = _gpu_graph(n, r, G, R, 1, causal, 41)
    rp, cols = _check_csr(orc, g, n, r, G, R, 1, causal, 41)
    shape = (1, 2, n, d)
    q = make_tensor(shape, 91, torch.bfloat16)
    k = make_tensor(shape, 92, torch.bfloat16)
    v = make_tensor(shape, 93, torch.bfloat16)
    q[0, 0] = 0
    q[0, 0, :, 0] = 16.0
    k[0, 0] = 0
    k[0, 0, 900, 0] = 32.0            # score 64 for key 900, 0 for every other key
    z = sah.attn(q.to(DEV), k.to(DEV), v.to(DEV), g, 5, 0.1)
    A = sah.scores_softmax(q.to(DEV), k.to(DEV), g)
    z_h, A_h = _as64(z), _as64(A)
    rpa, ca = np.asarray(rp[0]), np.asarray(cols[0])
    rows900 = np.repeat(np.arange(n), np.diff(rpa))[ca == 900]
    far = [i for i in rows900 if abs(i - 900) > r and i not in G]
    assert far, "key 900 must be a random neighbour of some row"
    for h in range(2):
        A_ref = orc.scores_softmax(_as64(q[0, h]), _as64(k[0, h]), rp[0], cols[0])
        A_csr = _a_csr(g, A_h, 0, h, 2, 0, rp, cols)
        assert np.all(np.abs(A_csr - A_ref) <= 2.0 ** -8 * A_ref + 1e-6), h
        ref = orc.attn(_as64(q[0, h]), _as64(k[0, h]), _as64(v[0, h]), rp[0], cols[0], 5, 0.1)
        pu.assert_z_close(z_h[0, h], ref, "bf16", f"attn h={h}", 5, 0.1)


def test_generic_scores_far_maximum_f32(orc):
    """fp32 (generic kernels): the whole path's single score pass, shifted by
    each row's own score, is redone with the exact maximum for rows whose
    weights would pass 2^64 (head 0); head 1 has ordinary inputs."""
    n, r, G, R = 600, 10, [0, 300], 24
    g = _gpu_graph(n, r, G, R, 1, False, 43)
    rp, cols = _check_csr(orc, g, n, r, G, R, 1, False, 43)
    shape = (1, 2, n, 32)
    q = make_tensor(shape, 94, torch.float32)
    k = make_tensor(shape, 95, torch.float32)
    v = make_tensor(shape, 96, torch.float32)
    q[0, 0] = 0
    q[0, 0, :, 0] = 16.0
    k[0, 0] = 0
    k[0, 0, 450, 0] = 45.0            # score 127 for key 450, 0 for every other key
    z = _as64(sah.attn(q.to(DEV), k.to(DEV), v.to(DEV), g, 5, 0.1))
    for h in range(2):
        ref = orc.attn(_as64(q[0, h]), _as64(k[0, h]), _as64(v[0, h]), rp[0], cols[0], 5, 0.1)
        pu.assert_z_close(z[0, h], ref, "f32", f"attn h={h}", 5, 0.1)


# Rows longer than 1024 slots go to the generic kernels' long-row companions
# (one workgroup per row): global rows of long sequences and, in a dense
# imported graph, every row.
LONG_ROW_CASES = [
    # id, graph maker (orc -> (graph, row_ptrs, cols)), B, H, d, dtype, K, alpha
    ("globals_f32_d64", lambda orc: (sah.build_graph(2500, 8, [0, 1, 1234, 2499], 5, 1, False, 9),
                                      *orc.graph(2500, 8, [0, 1, 1234, 2499], 5, 1, False, 9)),
     2, 2, 64, torch.float32, 3, 0.1),
    ("globals_causal_bf16_d128", lambda orc: (sah.build_graph(2100, 4, [0, 700, 2099], 3, 2, True, 4),
                                              *orc.graph(2100, 4, [0, 700, 2099], 3, 2, True, 4)),
     2, 1, 128, torch.bfloat16, 2, 0.3),
    ("dense_imported_f32_d16", lambda orc: (sah.graph_from_csr(
        1100, np.arange(1101, dtype=np.int64)[None, :] * 1100, [np.tile(np.arange(1100, dtype=np.int32), 1100)]),
        np.arange(1101, dtype=np.int64)[None, :] * 1100, [np.tile(np.arange(1100, dtype=np.int32), 1100)]),
     1, 2, 16, torch.float32, 2, 0.1),
]


@pytest.mark.parametrize("case", LONG_ROW_CASES, ids=lambda c: c[0])
def test_generic_long_rows(orc, case):
    name, make, B, H, d, tdt, K, alpha = case
    print(f"\n[long rows] {name}", flush=True)
    g, rp, cols = make(orc)
    ng = g.num_graphs
    shape = (B, H, g.n, d)
    q = make_tensor(shape, 81, tdt)
    k = make_tensor(shape, 82, tdt)
    v = make_tensor(shape, 83, tdt)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    A = sah.scores_softmax(qd, kd, g)
    z = sah.attn(qd, kd, vd, g, K, alpha)
    zs = sah.diffuse(A, vd, g, K, alpha)
    torch.cuda.synchronize()
    A_h, z_h, zs_h = _as64(A), _as64(z), _as64(zs)
    dt = pu.dtype_name(tdt)
    a_tol = 1e-5 if dt == "f32" else 2.0 ** -8 + 1e-5
    for b in range(B):
        gr = 0 if ng == 1 else b
        lens = np.diff(rp[gr])
        assert lens.max() > 1024, "the case must have long rows"
        for h in range(H):
            A_ref = orc.scores_softmax(_as64(q[b, h]), _as64(k[b, h]), rp[gr], cols[gr],
                                       pu.oracle_threads())
            A_got = _a_csr(g, A_h, b, h, H, gr, rp, cols)
            assert np.all(np.abs(A_got - A_ref) <= a_tol * np.maximum(A_ref, 1e-30) + 1e-12), (b, h)
            ref = orc.attn(_as64(q[b, h]), _as64(k[b, h]), _as64(v[b, h]), rp[gr], cols[gr], K,
                           alpha, pu.oracle_threads())
            pu.assert_z_close(z_h[b, h], ref, dt, f"{name} attn b={b} h={h}", K, alpha)
            ref_s = orc.diffuse(A_got, _as64(v[b, h]), rp[gr], cols[gr], K, alpha,
                                pu.oracle_threads())
            pu.assert_z_close(zs_h[b, h], ref_s, dt, f"{name} diffuse b={b} h={h}", K, alpha)


# fp32 row kernels with the window and global key rows in LDS (built graphs,
# d = 64, n > 1024, at least 1024 groups of 64 rows): global rows eight at a
# time in the diffusion step, the long-row companion in the score pass.
ROWS_F32_CASES = [
    # n, r, G, R, causal, B, H
    (2048, 10, [0, 1024, 2047], 24, False, 1, 32),
    (1100, 40, list(range(0, 1100, 50)), 30, True, 2, 30),
    (1300, 70, list(range(13)) + [650, 1299], 40, False, 4, 16),
    # no globals, n not a multiple of 16
    (2051, 20, [], 12, False, 1, 33),
    (1057, 33, [], 9, True, 1, 64),
]


@pytest.mark.parametrize("case", ROWS_F32_CASES, ids=lambda c: f"n{c[0]}r{c[1]}g{len(c[2])}c{int(c[4])}")
def test_rows_f32_kernels(orc, case):
    n, r, G, R, causal, B, H = case
    print(f"\n[rows f32] n={n} r={r} g={len(G)} R={R} causal={causal} B={B} H={H}", flush=True)
    g = _gpu_graph(n, r, G, R, 1, causal, 61)
    rp, cols = _check_csr(orc, g, n, r, G, R, 1, causal, 61)
    assert B * H * -(-n // 64) >= 1024
    shape = (B, H, n, 64)
    q, k, v = (make_tensor(shape, 71 + t, torch.float32) for t in range(3))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    z = sah.attn(qd, kd, vd, g, 3, 0.1)
    A = sah.scores_softmax(qd, kd, g)
    zs = sah.diffuse(A, vd, g, 3, 0.1)
    torch.cuda.synchronize()
    z_h, zs_h, A_h = _as64(z), _as64(zs), _as64(A)
    for b, h in {(0, 0), (0, H - 1), (B - 1, H // 2), (B - 1, 1)}:
        ref = orc.attn(_as64(q[b, h]), _as64(k[b, h]), _as64(v[b, h]), rp[0], cols[0], 3, 0.1,
                       pu.oracle_threads())
        pu.assert_z_close(z_h[b, h], ref, "f32", f"attn b={b} h={h}", 3, 0.1)
        A_got = _a_csr(g, A_h, b, h, H, 0, rp, cols)
        ref_s = orc.diffuse(A_got, _as64(v[b, h]), rp[0], cols[0], 3, 0.1, pu.oracle_threads())
        pu.assert_z_close(zs_h[b, h], ref_s, "f32", f"diffuse b={b} h={h}", 3, 0.1)


def test_rows_f32_far_maximum(orc):
    """The fp32 row score kernel's single pass, shifted by each row's own
    score, is redone with the exact maximum for rows whose weights would
    pass 2^64 (head 0); the other heads have ordinary inputs."""
    n, r, G, R, B, H = 2048, 10, [0, 1024], 24, 1, 32
    g = _gpu_graph(n, r, G, R, 1, False, 43)
    rp, cols = _check_csr(orc, g, n, r, G, R, 1, False, 43)
    shape = (B, H, n, 64)
    q, k, v = (make_tensor(shape, 94 + t, torch.float32) for t in range(3))
    q[0, 0] = 0
    q[0, 0, :, 0] = 16.0
    k[0, 0] = 0
    k[0, 0, 450, 0] = 45.0            # score 90 for key 450, 0 for every other key
    z = _as64(sah.attn(q.to(DEV), k.to(DEV), v.to(DEV), g, 5, 0.1))
    for h in (0, 1, 31):
        ref = orc.attn(_as64(q[0, h]), _as64(k[0, h]), _as64(v[0, h]), rp[0], cols[0], 5, 0.1)
        pu.assert_z_close(z[0, h], ref, "f32", f"attn h={h}", 5, 0.1)


def _slot_classes(g, gr, n, r, G, causal):
    """Class of every weight slot of graph gr: 0 window, 1 global column,
    2 random, 3 global row, -1 padding."""
    rows, sc = g.copy_slots(gr)
    rows = np.maximum(rows, 0)
    Gs = np.zeros(n, dtype=bool)
    Gs[list(G)] = True
    lo = np.maximum(rows - r, 0)
    hi = np.minimum(rows + r, n - 1)
    cls = np.full(len(sc), 2, dtype=np.int64)
    cls[(sc >= lo) & (sc <= hi)] = 0
    cls[(sc >= 0) & Gs[np.maximum(sc, 0)] & ~((sc >= lo) & (sc <= hi))] = 1
    cls[Gs[rows]] = 3
    cls[sc < 0] = -1
    return cls


@pytest.mark.parametrize("name", ["mlm4096_bf16", "long16k_bf16"])
def test_fast_diffusion_by_segment(orc, name):
    """One step, alpha = 0, with A restricted to one class of slots: isolates
    the window, global-column, random and global-row parts of the kernel.
    Both sides use the same stored bf16 weights and V, so the bound is the
    output's bf16 rounding (2^-8 relative) plus fp32 accumulation over at
    most n terms (1e-4 absolute)."""
    w = WORKLOADS[name]
    B, H = 1, 2
    g = _gpu_graph(w.n, w.radius, w.global_idx, w.num_random, 1, w.causal, w.graph_seed)
    rp, cols = _check_csr(orc, g, w.n, w.radius, w.global_idx, w.num_random, 1, w.causal,
                          w.graph_seed)
    cls = _slot_classes(g, 0, w.n, w.radius, w.global_idx, w.causal)
    q = make_tensor((B, H, w.n, 64), 5, torch.bfloat16).to(DEV)
    k = make_tensor((B, H, w.n, 64), 6, torch.bfloat16).to(DEV)
    v = make_tensor((B, H, w.n, 64), 7, torch.bfloat16).to(DEV)
    A = sah.scores_softmax(q, k, g)
    ns = g.slots[0]
    sr, sc = g.copy_slots(0)
    perm, _ = pu.slot_permutation(sr, sc, rp[0], cols[0])
    for c, cname in enumerate(["window", "global-col", "random", "global-row"]):
        mask = torch.tensor(np.tile(cls == c, B * H), device=DEV)
        Ac = torch.where(mask, A, torch.zeros_like(A))
        z = _as64(sah.diffuse(Ac, v, g, 1, 0.0))
        Ac_h = _as64(Ac)
        for h in range(H):
            ref = orc.diffuse(Ac_h[h * ns:(h + 1) * ns][perm], _as64(v[0, h]), rp[0], cols[0], 1,
                              0.0)
            err = np.abs(z[0, h] - ref)
            bad = np.argwhere(err > 2.0 ** -8 * np.abs(ref) + 1e-4)
            assert bad.size == 0, (f"{cname} h={h}: {len(bad)} bad, first rows/ch "
                                   f"{bad[:6].tolist()} max err {err.max():.3e}")


# ---------------------------------------------------------------------------
# General diffusion coefficients (eq. S.6 through A^K)
# ---------------------------------------------------------------------------

def _thetas(K):
    """PPR's coefficients at alpha 0.1, uniform ones, and A^K alone."""
    ppr = [0.1 * 0.9 ** k for k in range(K)] + [0.9 ** K]
    return {"ppr": ppr, "uniform": [1.0 / (K + 1)] * (K + 1), "last": [0.0] * K + [1.0]}


THETA_CASES = [
    # n, r, G, R, ng, causal, B, H, d, dtype
    (700, 20, list(range(0, 700, 7))[:70], 12, 2, False, 2, 2, 64, "bf16"),   # fast path
    (1100, 50, [0, 1, 2, 700, 1099], 40, 3, True, 3, 1, 64, "bf16"),          # fast, causal
    (300, 6, [0, 150], 9, 1, False, 2, 3, 64, "f32"),                          # generic
    (513, 16, [3, 200], 20, 1, False, 1, 2, 32, "bf16"),                       # generic, d 32
]


@pytest.mark.parametrize("case", THETA_CASES, ids=lambda c: f"n{c[0]}d{c[8]}{c[9]}c{int(c[5])}")
@pytest.mark.parametrize("K", [0, 1, 4])
def test_theta_small(orc, case, K):
    n, r, G, R, ngr, causal, B, H, d, dt = case
    ng = ngr if ngr in (1, B) else B
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    g = _gpu_graph(n, r, G, R, ng, causal, 37)
    rp, cols = _check_csr(orc, g, n, r, G, R, ng, causal, 37)
    shape = (B, H, n, d)
    q, k, v = (make_tensor(shape, 61 + i, tdt) for i in range(3))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    A = sah.scores_softmax(qd, kd, g)
    A_h = _as64(A)
    for tname, theta in _thetas(K).items():
        z = _as64(sah.attn_theta(qd, kd, vd, g, theta))
        zs = _as64(sah.diffuse_theta(A, vd, g, theta))
        for b in range(B):
            gr = 0 if ng == 1 else b
            for h in range(H):
                ref = orc.attn_theta(_as64(q[b, h]), _as64(k[b, h]), _as64(v[b, h]), rp[gr],
                                     cols[gr], theta)
                pu.assert_z_close(z[b, h], ref, dt, f"attn_theta {tname} b={b} h={h}", K, 0.0)
                A_csr = _a_csr(g, A_h, b, h, H, gr, rp, cols)
                ref_s = orc.diffuse_theta(A_csr, _as64(v[b, h]), rp[gr], cols[gr], theta)
                pu.assert_z_close(zs[b, h], ref_s, dt, f"diffuse_theta {tname} b={b} h={h}", K,
                                  0.0)
    if K == 0:   # theta = (1): Z = V exactly
        assert torch.equal(sah.attn_theta(qd, kd, vd, g, [1.0]), vd)


def test_theta_ppr_matches_recurrence():
    """PPR's coefficients through the nested form agree with the recurrence
    (the same operator, evaluated in another order)."""
    n, r, G, R = 700, 20, list(range(0, 700, 7))[:70], 12
    g = _gpu_graph(n, r, G, R, 2, False, 37)
    shape = (2, 2, n, 64)
    q, k, v = (make_tensor(shape, 71 + i, torch.bfloat16).to(DEV) for i in range(3))
    z1 = _as64(sah.attn(q, k, v, g, 5, 0.1))
    z2 = _as64(sah.attn_theta(q, k, v, g, _thetas(5)["ppr"]))
    for b in range(2):
        for h in range(2):
            pu.assert_z_close(z2[b, h], z1[b, h], "bf16", f"b={b} h={h}", 5, 0.1)


def test_theta_full_size(orc):
    """Headline workload, uniform coefficients over A^0 .. A^5, sampled pairs."""
    w = WORKLOADS["mlm4096_bf16"]
    print(f"\n[parity] theta {w.describe()}", flush=True)
    g = _gpu_graph(w.n, w.radius, w.global_idx, w.num_random, w.num_graphs, w.causal,
                   w.graph_seed)
    rp, cols = orc.graph(w.n, w.radius, w.global_idx, w.num_random, w.num_graphs, w.causal,
                         w.graph_seed)
    q, k, v = make_qkv(w)
    theta = _thetas(w.K)["uniform"]
    z = _as64(sah.attn_theta(q.to(DEV), k.to(DEV), v.to(DEV), g, theta))
    threads = pu.oracle_threads()
    for b, h in _samples(w.B, w.H)[:3]:
        gr = 0 if w.num_graphs == 1 else b
        ref = orc.attn_theta(_as64(q[b, h]), _as64(k[b, h]), _as64(v[b, h]), rp[gr], cols[gr],
                             theta, threads)
        e = pu.assert_z_close(z[b, h], ref, w.dtype, f"theta b={b} h={h}", w.K, 0.0)
        print(f"[parity] theta b={b} h={h} err={e:.3e} x tol", flush=True)


def test_theta_invalid():
    g = _gpu_graph(64, 2, [0], 3, 1, False, 5)
    x = make_tensor((1, 1, 64, 64), 1, torch.bfloat16).to(DEV)
    for bad in ([0.5, 0.4], [1.2, -0.2], [float("nan"), 1.0], [0.5, 0.5 + 1e-3]):
        with pytest.raises(sah.DiffuserError) as ei:
            sah.attn_theta(x, x, x, g, bad)
        assert ei.value.status_name == "DIFFUSER_ERR_INVALID_ARG", bad


# ---------------------------------------------------------------------------
# Evenly spaced extras ("w uni.")
# ---------------------------------------------------------------------------

EVEN_SPECS = [
    # n, r, G, R, num_graphs, causal
    (40, 2, [5, 30], 4, 1, False),
    (513, 16, [3, 200], 20, 2, False),
    (1100, 50, [0, 1, 2, 700, 1099], 40, 1, True),
    (64, 3, [0, 9, 50, 63], 100, 1, False),          # pool smaller than R
    (4096, 64, list(range(64)), 64, 8, False),       # headline shape
    (16384, 128, [k * 128 for k in range(128)], 128, 1, False),
]


@pytest.mark.parametrize("spec", EVEN_SPECS, ids=lambda s: f"n{s[0]}r{s[1]}R{s[3]}c{int(s[5])}")
def test_even_extras_csr_bitexact(orc, spec):
    n, r, G, R, ng, causal = spec
    g = sah.build_graph(n, r, G, R, ng, causal, 5, layout=sah.EXTRAS_EVEN)
    rp, cols = orc.graph(n, r, G, R, ng, causal, 5, layout=1)
    for gr in range(ng):
        grp, gcols = g.copy_csr(gr)
        assert np.array_equal(grp, rp[gr]), f"row_ptr mismatch in graph {gr}"
        assert np.array_equal(gcols, cols[gr]), f"col_idx mismatch in graph {gr}"
        sr, sc = g.copy_slots(gr)
        pu.slot_permutation(sr, sc, rp[gr], cols[gr])


@pytest.mark.parametrize("causal", [False, True])
def test_even_extras_attn(orc, causal):
    n, r, G, R = 1100, 20, [0, 1, 700], 40
    g = sah.build_graph(n, r, G, R, 1, causal, 5, layout=sah.EXTRAS_EVEN)
    rp, cols = orc.graph(n, r, G, R, 1, causal, 5, layout=1)
    shape = (1, 2, n, 64)
    q, k, v = (make_tensor(shape, 51 + i, torch.bfloat16) for i in range(3))
    z = _as64(sah.attn(q.to(DEV), k.to(DEV), v.to(DEV), g, 5, 0.1))
    for h in range(2):
        ref = orc.attn(_as64(q[0, h]), _as64(k[0, h]), _as64(v[0, h]), rp[0], cols[0], 5, 0.1)
        pu.assert_z_close(z[0, h], ref, "bf16", f"even h={h}")


def test_build_layout_invalid():
    with pytest.raises(sah.DiffuserError) as ei:
        sah.build_graph(64, 2, [0], 3, 1, False, 5, layout=2)
    assert ei.value.status_name == "DIFFUSER_ERR_INVALID_ARG"


# ---------------------------------------------------------------------------
# Backward of the whole path
# ---------------------------------------------------------------------------

def _assert_grad_close(got, ref, dtype, what):
    """f32: max error <= 1e-4 max|ref|; bf16: the output rounding (relative
    2^-9) plus fp32 accumulation: |err| <= 2^-8 |ref| + 1e-4 max|ref|."""
    scale = float(np.abs(ref).max(initial=0.0))
    err = np.abs(got - ref)
    if dtype == "f32":
        assert err.max(initial=0.0) <= 1e-4 * scale + 1e-7, (what, err.max(), scale)
    else:
        bound = 2.0 ** -8 * np.abs(ref) + 1e-4 * scale + 1e-7
        assert np.all(err <= bound), (what, float((err / bound).max()))


BACKWARD_CASES = [
    # n, r, G, R, ng, causal, B, H, d, dtype
    (300, 6, [0, 150], 9, 1, False, 2, 2, 64, "f32"),
    (513, 16, [3, 200], 20, 2, False, 2, 1, 64, "bf16"),
    (700, 20, list(range(0, 700, 7))[:70], 12, 1, True, 1, 2, 32, "bf16"),
    (257, 3, [], 5, 1, False, 1, 1, 128, "f32"),
    (129, 2, [64], 4, 1, True, 1, 1, 16, "f32"),
]


@pytest.mark.parametrize("case", BACKWARD_CASES, ids=lambda c: f"n{c[0]}d{c[8]}{c[9]}c{int(c[5])}")
@pytest.mark.parametrize("K,alpha", [(0, 0.1), (1, 0.3), (3, 0.1), (5, 0.0)])
def test_backward_small(orc, case, K, alpha):
    n, r, G, R, ngr, causal, B, H, d, dt = case
    ng = ngr if ngr in (1, B) else B
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    g = _gpu_graph(n, r, G, R, ng, causal, 43)
    rp, cols = orc.graph(n, r, G, R, ng, causal, 43)
    shape = (B, H, n, d)
    q, k, v, dz = (make_tensor(shape, 81 + i, tdt) for i in range(4))
    dq, dk, dv = (_as64(x) for x in sah.attn_backward(q.to(DEV), k.to(DEV), v.to(DEV), dz.to(DEV),
                                                      g, K, alpha))
    for b in range(B):
        gr = 0 if ng == 1 else b
        for h in range(H):
            rq, rk, rv = orc.attn_backward(_as64(q[b, h]), _as64(k[b, h]), _as64(v[b, h]),
                                           _as64(dz[b, h]), rp[gr], cols[gr], K, alpha)
            _assert_grad_close(dq[b, h], rq, dt, f"dQ b={b} h={h}")
            _assert_grad_close(dk[b, h], rk, dt, f"dK b={b} h={h}")
            _assert_grad_close(dv[b, h], rv, dt, f"dV b={b} h={h}")


def test_backward_imported_csr(orc):
    """An imported graph (any layout, here a dilated window)."""
    n, d = 200, 32
    rows = [sorted({i} | {j for j in range(i - 12, i + 13, 4) if 0 <= j < n}) for i in range(n)]
    rp = np.zeros(n + 1, dtype=np.int64)
    rp[1:] = np.cumsum([len(x) for x in rows])
    cols = np.concatenate([np.array(x, dtype=np.int32) for x in rows])
    g = sah.graph_from_csr(n, rp[None, :], cols)
    shape = (1, 2, n, d)
    q, k, v, dz = (make_tensor(shape, 91 + i, torch.float32) for i in range(4))
    dq, dk, dv = (_as64(x) for x in sah.attn_backward(q.to(DEV), k.to(DEV), v.to(DEV), dz.to(DEV),
                                                      g, 4, 0.2))
    for h in range(2):
        rq, rk, rv = orc.attn_backward(_as64(q[0, h]), _as64(k[0, h]), _as64(v[0, h]),
                                       _as64(dz[0, h]), rp, cols, 4, 0.2)
        _assert_grad_close(dq[0, h], rq, "f32", "dQ")
        _assert_grad_close(dk[0, h], rk, "f32", "dK")
        _assert_grad_close(dv[0, h], rv, "f32", "dV")


def test_backward_headline_shape(orc):
    """Headline graph and shape, two sampled (b, h) pairs; repeated calls are
    bitwise equal."""
    w = WORKLOADS["mlm4096_bf16"]
    print(f"\n[parity] backward {w.describe()}", flush=True)
    g = _gpu_graph(w.n, w.radius, w.global_idx, w.num_random, w.num_graphs, w.causal,
                   w.graph_seed)
    rp, cols = orc.graph(w.n, w.radius, w.global_idx, w.num_random, w.num_graphs, w.causal,
                         w.graph_seed)
    q, k, v = make_qkv(w)
    dz = make_tensor(q.shape, 7, torch.bfloat16)
    args = (q.to(DEV), k.to(DEV), v.to(DEV), dz.to(DEV), g, w.K, w.alpha)
    out = sah.attn_backward(*args)
    again = sah.attn_backward(*args)
    for x, y in zip(out, again):
        assert torch.equal(x, y)
    dq, dk, dv = (_as64(x) for x in out)
    for b, h in [(0, 0), (w.B - 1, w.H - 1)]:
        gr = 0 if w.num_graphs == 1 else b
        rq, rk, rv = orc.attn_backward(_as64(q[b, h]), _as64(k[b, h]), _as64(v[b, h]),
                                       _as64(dz[b, h]), rp[gr], cols[gr], w.K, w.alpha)
        _assert_grad_close(dq[b, h], rq, "bf16", f"dQ b={b} h={h}")
        _assert_grad_close(dk[b, h], rk, "bf16", f"dK b={b} h={h}")
        _assert_grad_close(dv[b, h], rv, "bf16", f"dV b={b} h={h}")
        print(f"[parity] backward b={b} h={h} ok", flush=True)


BACKWARD_ROWS_CASES = [
    # n, r, G, R, ng, causal, B, H, dtype, K, alpha: enough 64-row groups
    # (B H n / 64 >= 1024) for the LDS-window state kernels, global rows
    # first, inside and last
    (2048, 32, [0, 5, 1000, 2047], 24, 1, False, 1, 32, "f32", 5, 0.1),
    (2048, 40, list(range(0, 2048, 64)), 16, 2, True, 2, 16, "bf16", 3, 0.2),
    (2056, 24, [7, 2055], 10, 1, False, 1, 32, "bf16", 4, 0.0),
    # random weights in groups past the row segments (n > 4576)
    (6000, 16, [0, 2999, 5999], 12, 1, False, 1, 12, "f32", 2, 0.1),
    # no globals, n not a multiple of 16
    (2051, 20, [], 8, 1, False, 1, 33, "f32", 3, 0.1),
    (2051, 12, [], 6, 1, True, 1, 33, "bf16", 2, 0.3),
]


@pytest.mark.parametrize("case", BACKWARD_ROWS_CASES,
                         ids=lambda c: f"n{c[0]}{c[8]}c{int(c[5])}K{c[9]}")
def test_backward_rows_states(orc, case):
    """On built d = 64 graphs with enough rows the recomputed fp32 states
    and (bidirectional graphs) the transposed products come from the
    LDS-window step kernels; sampled (b, h) pairs against the oracle's
    chain rule."""
    n, r, G, R, ng, causal, B, H, dt, K, alpha = case
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    print(f"\n[parity] backward rows n={n} B={B} H={H} {dt} causal={causal} K={K}", flush=True)
    g = _gpu_graph(n, r, G, R, ng, causal, 61)
    rp, cols = orc.graph(n, r, G, R, ng, causal, 61)
    shape = (B, H, n, 64)
    q, k, v, dz = (make_tensor(shape, 121 + i, tdt) for i in range(4))
    dq, dk, dv = (_as64(x) for x in sah.attn_backward(q.to(DEV), k.to(DEV), v.to(DEV), dz.to(DEV),
                                                      g, K, alpha))
    for b, h in [(0, 0), (B - 1, H // 2), (B - 1, H - 1)]:
        gr = 0 if ng == 1 else b
        rq, rk, rv = orc.attn_backward(_as64(q[b, h]), _as64(k[b, h]), _as64(v[b, h]),
                                       _as64(dz[b, h]), rp[gr], cols[gr], K, alpha)
        _assert_grad_close(dq[b, h], rq, dt, f"dQ b={b} h={h}")
        _assert_grad_close(dk[b, h], rk, dt, f"dK b={b} h={h}")
        _assert_grad_close(dv[b, h], rv, dt, f"dV b={b} h={h}")


# ---------------------------------------------------------------------------
# One layer around the path (projections in, head concatenation and
# output projection out)
# ---------------------------------------------------------------------------

LAYER_CASES = [
    # n, r, G, R, ng, B, H, d, d_model, dtype
    (300, 6, [0, 150], 9, 1, 2, 2, 64, 96, "f32"),
    (513, 16, [3, 200], 20, 2, 2, 3, 64, 128, "bf16"),
    (700, 20, list(range(0, 700, 7))[:70], 12, 1, 1, 4, 32, 64, "bf16"),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=lambda c: f"n{c[0]}H{c[6]}d{c[7]}{c[9]}")
def test_layer_forward(orc, case):
    n, r, G, R, ngr, B, H, d, dm, dt = case
    ng = ngr if ngr in (1, B) else B
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    g = _gpu_graph(n, r, G, R, ng, False, 47)
    rp, cols = orc.graph(n, r, G, R, ng, False, 47)
    x = make_tensor((B, n, dm), 101, tdt)
    wq = make_tensor((dm, 3 * H * d), 102, tdt, scale=dm ** -0.5)
    wo = make_tensor((H * d, dm), 103, tdt, scale=(H * d) ** -0.5)
    y = _as64(sah.layer_forward(x.to(DEV), wq.to(DEV), wo.to(DEV), g, H, 5, 0.1))
    ref = orc.layer_forward(_as64(x), _as64(wq), _as64(wo), H, rp, cols, 5, 0.1,
                            round_bf16=(dt == "bf16"))
    # Y = Zc W_o: a per-element bound from the bound on Z, carried through
    # |W_o| column sums, plus one output rounding.
    colsum = np.abs(_as64(wo)).sum(axis=0)
    if dt == "f32":
        zc_mag = np.abs(ref).max()
        bound = 1e-4 * max(zc_mag, 1.0) * np.ones_like(ref) + 1e-6
    else:
        bound = pu.bf16_tolerance(5, 0.1) * colsum[None, None, :] + 2.0 ** -8 * np.abs(ref) + 1e-6
    err = np.abs(y - ref)
    assert np.all(err <= bound), float((err / bound).max())
