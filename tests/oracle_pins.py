"""Pins of the CPU oracle to facts outside itself.

Every check here compares the oracle with something it does not compute:
values printed on the pages (``tests/golden``), closed forms, invariants the
mathematics fixes, a textbook dense routine, or brute force on tiny inputs.
Each function takes an ``oracle.Oracle`` and raises AssertionError on a
mismatch, so the same checks run against the real oracle
(``test_oracle_pins.py``) and against deliberately broken builds of it
(``test_oracle_mutants.py``).
"""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def golden_dict(name):
    return {r[0]: r[1:] for r in read_golden(name)}


# --------------------------------------------------------------------------
# Set definitions written out directly (window eq. 5, globals eq. 12).
# --------------------------------------------------------------------------

def window_set(n, r, i):
    return set(range(max(0, i - r), min(n - 1, i + r) + 1))


def csr_rows(row_ptr, cols):
    return [cols[row_ptr[i]:row_ptr[i + 1]] for i in range(len(row_ptr) - 1)]


# --------------------------------------------------------------------------
# Random draws
# --------------------------------------------------------------------------

def pin_splitmix64(o):
    """Draw t of row 0, graph 0 is SplitMix64(seed=0)'s output t+1."""
    want = [int(r[0], 16) for r in read_golden("splitmix64_seed0.txt")]
    got = [o.draw(0, 0, 1, 0, t) for t in range(3)]
    assert got == want, (got, want)


# --------------------------------------------------------------------------
# Graph pins
# --------------------------------------------------------------------------

def pin_edge_counts_8pos(o):
    for n, r, gl, edges in read_golden("edge_counts_8pos.txt"):
        g = [] if gl == "-" else [int(x) for x in gl.split(",")]
        rp, _ = o.graph(int(n), int(r), g, 0)
        assert int(rp[0, -1]) == int(edges), (n, r, gl, int(rp[0, -1]), edges)


def pin_window_closed_form(o):
    """|E_local| = n(2r+1) - r(r+1) for n >= 2r+1; r >= n-1 gives n^2."""
    for n in (1, 2, 3, 5, 8, 13, 40, 97):
        for r in (0, 1, 2, 3, 7, 20, 48):
            rp, _ = o.graph(n, r, [], 0)
            nnz = int(rp[0, -1])
            if n >= 2 * r + 1:
                assert nnz == n * (2 * r + 1) - r * (r + 1), (n, r, nnz)
            if r >= n - 1:
                assert nnz == n * n, (n, r, nnz)


def _degree_formula(n, r, G, R, i):
    """Degree of row i from set sizes: n for a global row, else
    |W(i)| + |G minus W(i)| + min(R, n - |W(i) u G|)."""
    if i in G:
        return n
    w = window_set(n, r, i)
    gx = len(G - w)
    pool = n - len(w) - gx
    return len(w) + gx + min(R, pool)


def pin_degrees(o, cases=None):
    if cases is None:
        cases = [
            (64, 3, [0, 17, 63], 5, 2),
            (100, 10, [5, 6, 7, 50], 30, 1),
            (37, 4, [], 40, 1),          # pool smaller than the budget
            (50, 0, [10], 49, 1),        # r = 0, budget above the pool
            (300, 16, [0, 150], 8, 3),
        ]
    for n, r, G, R, ng in cases:
        rp, _ = o.graph(n, r, G, R, ng, False, 7)
        Gs = set(G)
        for gr in range(ng):
            deg = np.diff(rp[gr])
            want = np.array([_degree_formula(n, r, Gs, R, i) for i in range(n)])
            assert np.array_equal(deg, want), (n, r, G, R, gr)


def pin_row_structure(o):
    """Rows ascending without duplicates; self, window and globals present;
    random extras outside window and globals; causal graph is the
    bidirectional graph filtered to j <= i; seeds and graphs differ."""
    n, r, G, R = 200, 5, [0, 3, 99, 150], 12
    Gs = set(G)
    rp, cols = o.graph(n, r, G, R, 2, False, 11)
    rpc, colsc = o.graph(n, r, G, R, 2, True, 11)
    for gr in range(2):
        rows = csr_rows(rp[gr], cols[gr])
        rowsc = csr_rows(rpc[gr], colsc[gr])
        for i, row in enumerate(rows):
            assert np.all(np.diff(row) > 0), i
            s = set(row.tolist())
            assert i in s
            if i in Gs:
                assert s == set(range(n))
            else:
                assert window_set(n, r, i) <= s and Gs <= s
                extra = s - window_set(n, r, i) - Gs
                assert i not in extra and len(extra) == R
            want_c = sorted(j for j in s if j <= i)
            assert rowsc[i].tolist() == want_c, i
    # determinism and variation
    rp2, cols2 = o.graph(n, r, G, R, 2, False, 11)
    assert all(np.array_equal(a, b) for a, b in zip(cols, cols2))
    assert not np.array_equal(cols[0], cols[1])           # per-graph draws differ
    _, cols3 = o.graph(n, r, G, R, 1, False, 12)
    assert not np.array_equal(cols[0], cols3[0])           # per-seed draws differ


def pin_random_uniform(o):
    """Random extras are uniform over the pool: chi-square over column
    position for a window-free, global-free graph (pool = all j != i)."""
    n, R = 64, 8
    counts = np.zeros(n)
    ng = 200
    rp, cols = o.graph(n, 0, [], R, ng, False, 5)
    for gr in range(ng):
        for i, row in enumerate(csr_rows(rp[gr], cols[gr])):
            for j in row:
                if j != i:
                    counts[j] += 1
    expected = ng * R  # each column is in n-1 pools, chosen w.p. R/(n-1)
    chi2 = float(((counts - expected) ** 2 / expected).sum())
    # 63 degrees of freedom: the 1e-6 tail is far above 140
    assert chi2 < 140.0, chi2


# --------------------------------------------------------------------------
# Softmax pins
# --------------------------------------------------------------------------

def pin_softmax_8pos(o):
    g = golden_dict("softmax_8pos.txt")
    rp, cols = o.graph(8, 1, [], 0)
    rp, cols = rp[0], cols[0]
    w = np.array([float(x) for x in g["weights"]])
    for d in (1, 4):
        # score ln2 on the self edge of position 4 (index 3), 0 on its neighbours
        Q = np.zeros((8, d)); K = np.zeros((8, d))
        Q[3, 0] = math.sqrt(d)
        K[3, 0] = float(g["scores"][1])
        A = o.scores_softmax(Q, K, rp, cols)
        row = A[rp[3]:rp[4]]
        assert cols[rp[3]:rp[4]].tolist() == [2, 3, 4]
        assert np.allclose(row, w, rtol=0, atol=1e-15), (d, row)
    V = np.zeros((8, 2))
    V[2] = [float(x) for x in g["v3"]]
    V[3] = [float(x) for x in g["v4"]]
    V[4] = [float(x) for x in g["v5"]]
    Z = o.diffuse(A, V, rp, cols, 1, 0.0)
    assert np.allclose(Z[3], [float(x) for x in g["o4"]], rtol=0, atol=1e-15), Z[3]


def pin_row_sums(o):
    rng = np.random.default_rng(3)
    n, d = 150, 8
    rp, cols = o.graph(n, 4, [0, 75], 6, 1, False, 3)
    Q = rng.normal(size=(n, d)) * 3
    K = rng.normal(size=(n, d)) * 3
    A = o.scores_softmax(Q, K, rp[0], cols[0])
    sums = np.add.reduceat(A, rp[0][:-1])
    assert np.all(A > 0) and np.allclose(sums, 1.0, rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# Diffusion pins
# --------------------------------------------------------------------------

def pin_three_token(o):
    g = golden_dict("diffusion_3token.txt")
    A_dense = np.array([[float(x) for x in g[f"A_row{i}"]] for i in range(3)])
    rp = np.array([0, 2, 4, 5], dtype=np.int64)
    cols = np.array([0, 1, 1, 2, 2], dtype=np.int32)
    A = np.array([A_dense[i, j] for i in range(3) for j in cols[rp[i]:rp[i + 1]]])
    Z = o.diffuse(A, np.eye(3), rp, cols, int(g["K"][0]), float(g["alpha"][0]))
    want = [float(x) for x in g["Z2_row0_coeffs"]]
    assert np.allclose(Z[0], want, rtol=0, atol=1e-15), Z[0]


def pin_expansion_coefficients(o):
    """With A a cyclic shift, A^k e_0 are distinct unit vectors, so row 0 of
    Z_K for V = I lists the coefficient of each power A^k directly."""
    g = golden_dict("ppr_coeffs_k5.txt")
    K, alpha = int(g["K"][0]), float(g["alpha"][0])
    n = K + 2
    rp = np.arange(n + 1, dtype=np.int64)
    cols = ((np.arange(n) + 1) % n).astype(np.int32)      # A[i, i+1] = 1
    Z = o.diffuse(np.ones(n), np.eye(n), rp, cols, K, alpha)
    want = [float(x) for x in g["coeffs"]] + [0.0] * (n - K - 1)
    assert np.allclose(Z[0], want, rtol=0, atol=1e-15), Z[0]
    assert abs(sum(want) - 1.0) < 1e-15


def _dense_A(rp, cols, vals, n):
    A = np.zeros((n, n))
    for i in range(n):
        A[i, cols[rp[i]:rp[i + 1]]] = vals[rp[i]:rp[i + 1]]
    return A


def pin_finite_expansion(o):
    """Z_K = [(1-a)^K A^K + a sum_{i<K} (1-a)^i A^i] V by dense matrix powers."""
    rng = np.random.default_rng(9)
    n, d = 40, 5
    rp, cols = o.graph(n, 2, [7], 3, 1, False, 9)
    rp, cols = rp[0], cols[0]
    Q, Kx, V = (rng.normal(size=(n, d)) for _ in range(3))
    A = o.scores_softmax(Q, Kx, rp, cols)
    Ad = _dense_A(rp, cols, A, n)
    for K in (0, 1, 2, 5, 9):
        for alpha in (0.0, 0.05, 0.1, 0.3, 1.0):
            M = (1 - alpha) ** K * np.linalg.matrix_power(Ad, K)
            for i in range(K):
                M = M + alpha * (1 - alpha) ** i * np.linalg.matrix_power(Ad, i)
            Z = o.diffuse(A, V, rp, cols, K, alpha)
            assert np.allclose(Z, M @ V, rtol=0, atol=1e-12), (K, alpha)


def pin_dense_brute_force(o):
    """Dense masked softmax (mask 0 / -inf, eqs. 2-4) plus dense diffusion on
    tiny n; the mask comes from the set definitions, the random columns
    from the CSR's entries outside window and globals."""
    rng = np.random.default_rng(21)
    for n, r, G, R, causal in [(16, 1, [3], 2, False), (33, 3, [0, 32], 4, False),
                               (24, 2, [5, 11], 3, True), (9, 0, [], 0, False),
                               (12, 20, [], 0, True)]:
        d = 6
        rp, cols = o.graph(n, r, G, R, 1, causal, 4)
        rp, cols = rp[0], cols[0]
        allowed = np.zeros((n, n), dtype=bool)
        for i in range(n):
            if i in G:
                allowed[i, :] = True
            else:
                allowed[i, list(window_set(n, r, i))] = True
                allowed[i, G] = True
                row = set(cols[rp[i]:rp[i + 1]].tolist())
                rnd = row - window_set(n, r, i) - set(G)
                allowed[i, sorted(rnd)] = True
            if causal:
                allowed[i, i + 1:] = False
        # the oracle's structure must equal the mask (random part is its own)
        got = np.zeros((n, n), dtype=bool)
        for i in range(n):
            got[i, cols[rp[i]:rp[i + 1]]] = True
        assert np.array_equal(got, allowed), (n, r, G, R, causal)
        Q, Kx, V = (rng.normal(size=(n, d)) for _ in range(3))
        S = Q @ Kx.T / math.sqrt(d) + np.where(allowed, 0.0, -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        A = o.scores_softmax(Q, Kx, rp, cols)
        assert np.allclose(_dense_A(rp, cols, A, n), P, rtol=0, atol=1e-14)
        K, alpha = 4, 0.2
        Z = V.copy()
        for _ in range(K):
            Z = (1 - alpha) * P @ Z + alpha * V
        assert np.allclose(o.diffuse(A, V, rp, cols, K, alpha), Z, rtol=0, atol=1e-12)


def pin_softmax_attention_reduction(o):
    """Complete graph, alpha = 0, K = 1 is ordinary softmax attention; alpha = 1
    or K = 0 returns V exactly."""
    rng = np.random.default_rng(5)
    n, d = 30, 8
    rp, cols = o.graph(n, n, [], 0)
    Q, Kx, V = (rng.normal(size=(n, d)) for _ in range(3))
    S = Q @ Kx.T / math.sqrt(d)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    A = o.scores_softmax(Q, Kx, rp[0], cols[0])
    assert np.allclose(o.diffuse(A, V, rp[0], cols[0], 1, 0.0), P @ V, rtol=0, atol=1e-13)
    assert np.array_equal(o.diffuse(A, V, rp[0], cols[0], 0, 0.1), V)
    assert np.array_equal(o.diffuse(A, V, rp[0], cols[0], 6, 1.0), V)


def pin_infinite_limit(o):
    """||Z_K - a (I - (1-a) A)^-1 V||_inf <= 2 (1-a)^K ||V||_inf, and Z_K reaches
    the linear-solve limit for large K."""
    rng = np.random.default_rng(13)
    n, d = 25, 4
    rp, cols = o.graph(n, 2, [12], 3, 1, False, 8)
    rp, cols = rp[0], cols[0]
    Q, Kx, V = (rng.normal(size=(n, d)) for _ in range(3))
    A = o.scores_softmax(Q, Kx, rp, cols)
    Ad = _dense_A(rp, cols, A, n)
    for alpha in (0.05, 0.1, 0.3):
        Zinf = alpha * np.linalg.solve(np.eye(n) - (1 - alpha) * Ad, V)
        for K in (1, 3, 5, 10):
            err = np.abs(o.diffuse(A, V, rp, cols, K, alpha) - Zinf).max()
            assert err <= 2 * (1 - alpha) ** K * np.abs(V).max() + 1e-12, (alpha, K, err)
        Z = o.diffuse(A, V, rp, cols, 600, alpha)
        assert np.allclose(Z, Zinf, rtol=0, atol=1e-9), alpha


def _perturbation_dependence(o, n, r, G, R, causal, K, alpha, p, seed=2):
    rng = np.random.default_rng(seed)
    d = 3
    rp, cols = o.graph(n, r, G, R, 1, causal, 6)
    rp, cols = rp[0], cols[0]
    Q, Kx, V = (rng.normal(size=(n, d)) for _ in range(3))
    A = o.scores_softmax(Q, Kx, rp, cols)
    Z0 = o.diffuse(A, V, rp, cols, K, alpha)
    V2 = V.copy()
    V2[p] += 1.0
    Z1 = o.diffuse(A, V2, rp, cols, K, alpha)
    return np.any(Z0 != Z1, axis=1)


def pin_causality(o):
    """Causal graph: changing V[p] leaves Z[i < p] bitwise unchanged."""
    for p in (0, 10, 31, 59):
        changed = _perturbation_dependence(o, 60, 3, [0, 20, 40], 4, True, 5, 0.1, p)
        assert not changed[:p].any(), p
        assert changed[p]


def pin_reach(o):
    """Window-only graph: Z[i] depends on V[p] iff |i - p| <= K r."""
    n, r, K, p = 80, 3, 4, 40
    changed = _perturbation_dependence(o, n, r, [], 0, False, K, 0.1, p)
    idx = np.arange(n)
    assert np.array_equal(changed, np.abs(idx - p) <= K * r), np.nonzero(changed)


def pin_two_hop_global(o):
    """Non-causal graph with a global token and K >= 2: every output depends
    on every input row; with K = 1 a far token does not."""
    n = 50
    for p in (3, 25, 49):
        assert _perturbation_dependence(o, n, 1, [20], 0, False, 2, 0.1, p).all(), p
    changed = _perturbation_dependence(o, n, 1, [20], 0, False, 1, 0.1, 45)
    assert not changed[0]


def pin_constant_fixed_point(o):
    """Constant V (every row the same) is a fixed point: Z_k = V."""
    rng = np.random.default_rng(17)
    n, d = 70, 4
    rp, cols = o.graph(n, 5, [0, 69], 7, 1, False, 1)
    Q, Kx = rng.normal(size=(n, d)), rng.normal(size=(n, d))
    A = o.scores_softmax(Q, Kx, rp[0], cols[0])
    V = np.tile(rng.normal(size=(1, d)), (n, 1))
    Z = o.diffuse(A, V, rp[0], cols[0], 7, 0.1)
    assert np.allclose(Z, V, rtol=0, atol=1e-13)


def pin_theta_printed_coefficients(o):
    """General coefficients (eq. S.6): with A a cyclic shift and V = I, row 0
    of sum_k theta_k A^k V lists theta itself; with the printed K = 5,
    alpha = 0.1 coefficients the operator equals the PPR recurrence."""
    g = golden_dict("ppr_coeffs_k5.txt")
    K, alpha = int(g["K"][0]), float(g["alpha"][0])
    theta = [float(x) for x in g["coeffs"]]
    n = K + 2
    rp = np.arange(n + 1, dtype=np.int64)
    cols = ((np.arange(n) + 1) % n).astype(np.int32)
    Z = o.diffuse_theta(np.ones(n), np.eye(n), rp, cols, theta)
    assert np.allclose(Z[0], theta + [0.0] * (n - K - 1), rtol=0, atol=1e-15), Z[0]
    rng = np.random.default_rng(11)
    m = 40
    rp, cols = o.graph(m, 2, [5, 30], 4, 1, False, 17)
    A = o.scores_softmax(rng.standard_normal((m, 8)), rng.standard_normal((m, 8)), rp[0],
                         cols[0])
    V = rng.standard_normal((m, 3))
    Zt = o.diffuse_theta(A, V, rp[0], cols[0], theta)
    Zp = o.diffuse(A, V, rp[0], cols[0], K, alpha)
    assert np.max(np.abs(Zt - Zp)) < 1e-12


def pin_theta_three_token(o):
    """The three-token example through the general form: theta = (alpha,
    alpha (1 - alpha), (1 - alpha)^2) for K = 2 gives the printed row."""
    g = golden_dict("diffusion_3token.txt")
    alpha = float(g["alpha"][0])
    A_dense = np.array([[float(x) for x in g[f"A_row{i}"]] for i in range(3)])
    rp = np.array([0, 2, 4, 5], dtype=np.int64)
    cols = np.array([0, 1, 1, 2, 2], dtype=np.int32)
    A = np.array([A_dense[i, j] for i in range(3) for j in cols[rp[i]:rp[i + 1]]])
    theta = [alpha, alpha * (1 - alpha), (1 - alpha) ** 2]
    Z = o.diffuse_theta(A, np.eye(3), rp, cols, theta)
    want = [float(x) for x in g["Z2_row0_coeffs"]]
    assert np.allclose(Z[0], want, rtol=0, atol=1e-15), Z[0]


def pin_theta_powers(o):
    """theta = e_k gives A^k V (dense matrix powers); theta = e_0 gives V
    exactly; mixtures are the same mixture of powers."""
    rng = np.random.default_rng(12)
    n = 24
    rp, cols = o.graph(n, 1, [7], 3, 1, False, 23)
    A = o.scores_softmax(rng.standard_normal((n, 4)), rng.standard_normal((n, 4)), rp[0],
                         cols[0])
    Ad = _dense_A(rp[0], cols[0], A, n)
    V = rng.standard_normal((n, 5))
    assert np.array_equal(o.diffuse_theta(A, V, rp[0], cols[0], [1.0]), V)
    for k in range(1, 5):
        th = [0.0] * k + [1.0]
        want = np.linalg.matrix_power(Ad, k) @ V
        assert np.max(np.abs(o.diffuse_theta(A, V, rp[0], cols[0], th) - want)) < 1e-12, k
    th = [0.2, 0.0, 0.5, 0.3]
    want = 0.2 * V + 0.5 * Ad @ Ad @ V + 0.3 * np.linalg.matrix_power(Ad, 3) @ V
    assert np.max(np.abs(o.diffuse_theta(A, V, rp[0], cols[0], th) - want)) < 1e-12


def _pool_ranks(n, r, G, rp, cols, i):
    """Pool of row i (positions outside its window and the globals) and the
    ranks in it of the row's extras."""
    lo, hi = max(0, i - r), min(n - 1, i + r)
    Gs = set(G)
    pool = [j for j in range(n) if (j < lo or j > hi) and j not in Gs]
    row = set(int(c) for c in cols[rp[i]:rp[i + 1]])
    extras = sorted(row - set(range(lo, hi + 1)) - Gs)
    where = {j: t for t, j in enumerate(pool)}
    return pool, [where[j] for j in extras]


def pin_even_extras(o):
    """Evenly spaced extras ("w uni."): min(R, P) of them; among the first m
    members of the pool there are exactly ceil(m R / P) (even spacing with
    the first member taken); the same for every seed and graph; the causal
    graph is the bidirectional one filtered to j <= i; degrees as for random
    extras."""
    for n, r, G, R in [(40, 2, [5, 30], 4), (33, 1, [], 7), (64, 3, [0, 9, 50, 63], 13),
                       (17, 4, [8], 20)]:
        rp2, cols2 = o.graph(n, r, G, R, 2, False, 3, layout=1)
        rp_b, cols_b = o.graph(n, r, G, R, 1, False, 99, layout=1)
        assert np.array_equal(rp2[0], rp2[1]) and np.array_equal(cols2[0], cols2[1])
        assert np.array_equal(rp2[0], rp_b[0]) and np.array_equal(cols2[0], cols_b[0])
        rp, cols = rp2[0], cols2[0]
        rpr, _ = o.graph(n, r, G, R, 1, False, 3, layout=0)
        assert np.array_equal(rp, rpr[0]), "degrees differ from the random layout"
        for i in range(n):
            if i in G:
                continue
            pool, ranks = _pool_ranks(n, r, G, rp, cols, i)
            P = len(pool)
            assert len(ranks) == min(R, P), (n, i)
            if P > R:
                for m in range(P + 1):
                    assert sum(t < m for t in ranks) == -(-m * R // P), (n, i, m)
        rpc, colsc = o.graph(n, r, G, R, 1, True, 3, layout=1)
        for i in range(n):
            want = [int(c) for c in cols[rp[i]:rp[i + 1]] if c <= i]
            assert [int(c) for c in colsc[0][rpc[0][i]:rpc[0][i + 1]]] == want, (n, i)


def pin_backward_finite_differences(o):
    """The gradients of sum(dZ * Z) match central differences of the oracle's
    own forward pass in every coordinate of Q, K and V (bidirectional graph
    with a global row; causal graph)."""
    rng = np.random.default_rng(21)
    for n, r, G, R, causal, K, alpha in [(24, 2, [5], 3, False, 3, 0.2),
                                         (20, 1, [0, 13], 4, True, 2, 0.1)]:
        rp, cols = o.graph(n, r, G, R, 1, causal, 31)
        rp, cols = rp[0], cols[0]
        Q, Kx, V, dZ = (rng.standard_normal((n, 3)) for _ in range(4))
        dQ, dK, dV = o.attn_backward(Q, Kx, V, dZ, rp, cols, K, alpha)

        def loss(q, k, v):
            return float((dZ * o.attn(q, k, v, rp, cols, K, alpha)).sum())

        h = 1e-6
        for which, grad in ((0, dQ), (1, dK), (2, dV)):
            for idx in np.ndindex(n, 3):
                args_p = [Q.copy(), Kx.copy(), V.copy()]
                args_m = [Q.copy(), Kx.copy(), V.copy()]
                args_p[which][idx] += h
                args_m[which][idx] -= h
                fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
                assert abs(fd - grad[idx]) < 1e-7 * max(1.0, abs(fd)), (which, idx, fd, grad[idx])


def pin_backward_special_cases(o):
    """alpha = 1 or K = 0 make Z = V: then dV = dZ and dQ = dK = 0 exactly."""
    rng = np.random.default_rng(22)
    rp, cols = o.graph(16, 1, [3], 2, 1, False, 4)
    Q, Kx, V, dZ = (rng.standard_normal((16, 4)) for _ in range(4))
    for K, alpha in ((3, 1.0), (0, 0.3)):
        dQ, dK, dV = o.attn_backward(Q, Kx, V, dZ, rp[0], cols[0], K, alpha)
        assert np.array_equal(dV, dZ) and not dQ.any() and not dK.any(), (K, alpha)


def pin_bf16_rounding(o):
    """Round to nearest even on bf16 (8 significant bits): ties go to the
    even significand."""
    import oracle as _oracle
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -7, -(1 + 2.0 ** -8 + 2.0 ** -12),
                  3.0e38, 2.0 ** -130])
    want = np.array([1.0, 1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -(1 + 2.0 ** -7), 226 * 2.0 ** 120,
                     2.0 ** -130])
    got = _oracle.round_bf16_rne(x)
    assert np.allclose(got, want, rtol=1e-7, atol=0), got


def pin_layer_identity(o):
    """With identity projections (d_model = H d, W_qkv = [I I I], W_o = I)
    the layer returns each head's attention on its own slice of X, placed
    back in its slice; consistent permutations of heads leave Y unchanged."""
    rng = np.random.default_rng(31)
    B, n, H, d = 2, 20, 3, 4
    D = H * d
    rp, cols = o.graph(n, 2, [4], 3, 1, False, 9)
    X = rng.standard_normal((B, n, D))
    W_qkv = np.concatenate([np.eye(D)] * 3, axis=1)
    Y = o.layer_forward(X, W_qkv, np.eye(D), H, rp, cols, 3, 0.2)
    for b in range(B):
        for h in range(H):
            xs = X[b, :, h * d:(h + 1) * d]
            want = o.attn(xs, xs, xs, rp[0], cols[0], 3, 0.2)
            assert np.max(np.abs(Y[b, :, h * d:(h + 1) * d] - want)) < 1e-13, (b, h)
    Wq = rng.standard_normal((D, 3 * H * d))
    Wo = rng.standard_normal((H * d, D))
    perm = [2, 0, 1]
    cols_perm = np.concatenate([np.arange(p * H * d + h * d, p * H * d + (h + 1) * d)
                                for p in range(3) for h in perm])
    rows_perm = np.concatenate([np.arange(h * d, (h + 1) * d) for h in perm])
    Y1 = o.layer_forward(X, Wq, Wo, H, rp, cols, 3, 0.2)
    Y2 = o.layer_forward(X, Wq[:, cols_perm], Wo[rows_perm], H, rp, cols, 3, 0.2)
    assert np.max(np.abs(Y1 - Y2)) < 1e-10


# --------------------------------------------------------------------------
# Block graph (BigBird, eq. 13) and dilated window (Longformer, eq. 11)
# --------------------------------------------------------------------------

def _key_block_count(N, h, gb, s, I):
    """Key blocks of query block I from set sizes: N for a global block,
    else |L u G| + min(s, N - |L u G|)."""
    if I < gb:
        return N
    base = set(range(max(0, I - h), min(N - 1, I + h) + 1)) | set(range(gb))
    return len(base) + min(s, N - len(base))


def pin_block_graph_example(o):
    g = golden_dict("bigbird_12blocks.txt")
    N, b, c, s, gb = (int(g[k][0]) for k in ("blocks", "block", "local", "random", "global"))
    n = N * b
    rp, cols, blocks = o.block_graph(n, b, c, s, gb, 1, 0)
    keys = blocks[0]
    I = int(g["example_query_block"][0])
    local = {int(x) for x in g["example_local"][0].split(",")}
    glob = {int(x) for x in g["example_global"][0].split(",")}
    assert local | glob <= set(keys[I]), keys[I]
    assert len(keys[I]) == 6
    deg = np.diff(rp[0])
    assert int(deg[I * b:(I + 1) * b].sum()) == int(g["pairs_ordinary_block"][0])
    assert int(deg[0:b].sum()) == int(g["pairs_global_block"][0])
    nnz = int(rp[0, -1])
    assert (N - gb) * int(g["pairs_ordinary_block"][0]) + gb * int(g["pairs_global_block"][0]) \
        == int(g["upper_bound"][0])
    assert nnz <= int(g["upper_bound"][0]) < int(g["full"][0]) == n * n
    want = sum(_key_block_count(N, (c - 1) // 2, gb, s, J) for J in range(N)) * b * b
    assert nnz == want, (nnz, want)


def pin_block_graph_structure(o):
    """Rows of one block are identical and ascending; each is a union of
    whole key blocks: the local blocks, the global blocks and exactly
    min(s, pool) distinct others; global query blocks read everything;
    seeds and graphs vary the draws."""
    cases = [(96, 8, 3, 2, 1), (128, 16, 1, 3, 0), (64, 8, 5, 9, 2), (64, 16, 9, 2, 1),
             (256, 16, 3, 4, 2)]
    for n, b, c, s, gb in cases:
        N, h = n // b, (c - 1) // 2
        rp, cols, blocks = o.block_graph(n, b, c, s, gb, 2, 5)
        for gr in range(2):
            rows = csr_rows(rp[gr], cols[gr])
            for I in range(N):
                ks = blocks[gr][I]
                want = np.concatenate([np.arange(J * b, (J + 1) * b) for J in ks])
                for i in range(I * b, (I + 1) * b):
                    assert np.array_equal(rows[i], want), (n, b, c, s, gb, i)
                assert np.all(np.diff(ks) > 0)
                assert len(ks) == _key_block_count(N, h, gb, s, I)
                if I < gb:
                    assert ks == list(range(N))
                else:
                    base = set(range(max(0, I - h), min(N - 1, I + h) + 1)) | set(range(gb))
                    assert base <= set(ks)
    n, b, c, s, gb = 256, 8, 3, 4, 1
    _, c1, _ = o.block_graph(n, b, c, s, gb, 2, 5)
    _, c2, _ = o.block_graph(n, b, c, s, gb, 2, 5)
    _, c3, _ = o.block_graph(n, b, c, s, gb, 1, 6)
    assert all(np.array_equal(x, y) for x, y in zip(c1, c2))
    assert not np.array_equal(c1[0], c1[1]) and not np.array_equal(c1[0], c3[0])


def pin_block_random_uniform(o):
    """Random key blocks are spread evenly over the pool: over many query
    blocks each pool block is picked about equally often."""
    n, b, c, s, gb = 4096, 4, 3, 8, 2
    N = n // b
    _, _, blocks = o.block_graph(n, b, c, s, gb, 1, 3)
    hits = np.zeros(N)
    for I in range(gb, N):
        base = set(range(max(0, I - 1), min(N - 1, I + 1) + 1)) | set(range(gb))
        for J in blocks[0][I]:
            if J not in base:
                hits[J] += 1
    inner = hits[gb + 8:N - 8]
    mean = (N - gb) * s / (N - gb - 3)
    assert abs(inner.mean() - mean) < 0.05 * mean, inner.mean()
    assert inner.std() < 3.5 * math.sqrt(mean), inner.std()


def pin_block_draws_golden(o):
    """Query block 0 of graph 0 (no global blocks, c = 1, seed 0) takes its
    random blocks from SplitMix64(seed 0)'s first outputs (the golden file),
    each mapped to a block by (u >> 32) N >> 32."""
    u = [int(r[0], 16) for r in read_golden("splitmix64_seed0.txt")]
    N, b = 1000, 4
    want = []
    for x in u:
        J = ((x >> 32) * N) >> 32
        if J != 0 and J not in want:
            want.append(J)
    want = sorted(want[:2])
    assert len(want) == 2
    _, _, blocks = o.block_graph(N * b, b, 1, 2, 0, 1, 0)
    assert blocks[0][0] == sorted([0] + want), (blocks[0][0], want)


def pin_token_draws_golden(o):
    """Random extras of the token graph straight from SplitMix64(seed 0)'s
    first outputs (the golden file): draw t of row i of graph b uses the
    counter ((b n + i) << 20) | t, so with seed = -(c << 20) gamma (mod 2^64)
    the row whose packed index is c replays outputs 1, 2, 3 of seed 0. Each
    output maps to column (u >> 32) n >> 32 and is kept unless it is in the
    row's window, a global position or already taken, in draw order.
    n = 1000, radius 20, global {431}, 2 extras: the outputs map to 883, 431
    (global, skipped) and 26, so the row is its window, 26, 431 and 883.
    Checked for row 0 of graph 0 (seed 0), row 1 of graph 0 and row 0 of
    graph 1 (the two packings of a nonzero index)."""
    u = [int(r[0], 16) for r in read_golden("splitmix64_seed0.txt")]
    n, r, G = 1000, 20, [431]
    cols = [((x >> 32) * n) >> 32 for x in u]
    assert cols == [883, 431, 26], cols
    gamma = 0x9E3779B97F4A7C15
    for b, i in ((0, 0), (0, 1), (1, 0)):
        c = b * n + i
        seed = (-(c << 20) * gamma) % (1 << 64)
        rp, cl = o.graph(n, r, G, 2, 2, False, seed)
        row = csr_rows(rp[b], cl[b])[i].tolist()
        want = sorted(set(range(0, i + r + 1)) | {26, 431, 883})
        assert row == want, (b, i, row, want)


def pin_dilated_example(o):
    for r, dl, pos, nb in read_golden("dilated_window.txt"):
        r, dl, i = int(r), int(dl), int(pos) - 1
        want = [int(x) - 1 for x in nb.split(",")]
        rp, cols = o.dilated_graph(40, r, dl, [])
        row = csr_rows(rp[0], cols[0])[i].tolist()
        assert row == want, (row, want)
        assert i - 1 not in row and i + 1 not in row


def pin_dilated_structure(o):
    """Step 1 is the contiguous window with globals (the token graph
    without random extras); with step delta and no globals every neighbour
    is congruent to the row mod delta and rows have at most 2r + 1 of them;
    global rows are full."""
    for n, r, G in ((50, 3, [0, 17]), (33, 0, []), (64, 5, [63])):
        rp1, c1 = o.dilated_graph(n, r, 1, G)
        rp2, c2 = o.graph(n, r, G, 0)
        assert np.array_equal(rp1[0], rp2[0]) and np.array_equal(c1[0], c2[0]), (n, r, G)
    n, r, dl = 100, 4, 7
    rp, cols = o.dilated_graph(n, r, dl, [])
    for i, row in enumerate(csr_rows(rp[0], cols[0])):
        assert len(row) <= 2 * r + 1 and i in row
        assert all((j - i) % dl == 0 and abs(j - i) <= r * dl for j in row), i
    rp, cols = o.dilated_graph(n, r, dl, [5, 60])
    rows = csr_rows(rp[0], cols[0])
    assert rows[5].tolist() == list(range(n)) and rows[60].tolist() == list(range(n))
    assert {5, 60} <= set(rows[30].tolist())


ALL_PINS = [
    pin_splitmix64, pin_edge_counts_8pos, pin_window_closed_form, pin_degrees,
    pin_row_structure, pin_random_uniform, pin_softmax_8pos, pin_row_sums,
    pin_three_token, pin_expansion_coefficients, pin_finite_expansion,
    pin_dense_brute_force, pin_softmax_attention_reduction, pin_infinite_limit,
    pin_causality, pin_reach, pin_two_hop_global, pin_constant_fixed_point,
    pin_theta_printed_coefficients, pin_theta_three_token, pin_theta_powers,
    pin_even_extras, pin_backward_finite_differences, pin_backward_special_cases,
    pin_bf16_rounding, pin_layer_identity, pin_block_graph_example, pin_block_graph_structure,
    pin_block_random_uniform, pin_block_draws_golden, pin_token_draws_golden, pin_dilated_example,
    pin_dilated_structure,
]
