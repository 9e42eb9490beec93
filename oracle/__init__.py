"""Diffuser CPU oracle -- TEST INFRASTRUCTURE ONLY.

Plain double-precision CPU implementation of the Diffuser attention-diffusion
path (graph, edge scores, edge softmax, K-step personalized-PageRank
diffusion), written in C (``oracle.c``) and reached through ctypes.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module. It shares no code with the HIP library.

Sources: "Diffuser" reading notes sections 2.1 (eqs. S.1-S.5), 2.2, 2.4
(eq. S.7), 2.5; "1.2.1 Static sparsity" sections 1, 1.1 (eq. 5), 1.2 (eqs. 11
and 12), 2 (eq. 13, the block graph); "038 BigBird" section 2 (union
neighbourhood).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

_lib = None


def build(out_path: str = LIB_PATH, src_path: str = SRC_PATH, extra_flags=()) -> str:
    """Compiles the oracle with gcc (plain -O2, no fast-math: summation order
    is part of the oracle's definition)."""
    tmp = out_path + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
           *extra_flags, src_path, "-o", tmp, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def _bind(lib):
    i64, i32, u64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64
    p = ctypes.c_void_p
    lib.oracle_mix64.restype = u64
    lib.oracle_mix64.argtypes = [u64]
    lib.oracle_draw.restype = u64
    lib.oracle_draw.argtypes = [u64, i64, i64, i64, i64]
    graph_args = [i64, i32, i32, p, i32, i32, i32, u64]
    lib.oracle_graph_nnz.restype = ctypes.c_int
    lib.oracle_graph_nnz.argtypes = graph_args + [p]
    lib.oracle_graph_build.restype = ctypes.c_int
    lib.oracle_graph_build.argtypes = graph_args + [p, p]
    lib.oracle_graph_nnz_layout.restype = ctypes.c_int
    lib.oracle_graph_nnz_layout.argtypes = graph_args + [i32, p]
    lib.oracle_graph_build_layout.restype = ctypes.c_int
    lib.oracle_graph_build_layout.argtypes = graph_args + [i32, p, p]
    for name in ("oracle_scores_softmax", "oracle_scores"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [p, p, i64, i32, p, p, p, i32]
    lib.oracle_diffuse.restype = ctypes.c_int
    lib.oracle_diffuse.argtypes = [p, p, i64, i32, p, p, i32, ctypes.c_double, p, i32]
    lib.oracle_attn_backward.restype = ctypes.c_int
    lib.oracle_attn_backward.argtypes = [p, p, p, p, i64, i32, p, p, i32, ctypes.c_double, p, p,
                                         p]
    lib.oracle_diffuse_theta.restype = ctypes.c_int
    lib.oracle_diffuse_theta.argtypes = [p, p, i64, i32, p, p, i32, p, p, i32]
    return lib


def round_bf16_rne(x):
    """Nearest bf16 value (ties to even) of each element, via its float32
    value, as float64."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def load(path: str = LIB_PATH):
    """Loads (building first if absent) the oracle library."""
    global _lib
    if path != LIB_PATH:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(path):
            build()
        _lib = _bind(ctypes.CDLL(path))
    return _lib


class OracleError(RuntimeError):
    pass


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(st: int, what: str):
    if st != 0:
        raise OracleError(f"{what} failed with status {st}")


class Oracle:
    """Thin numpy-facing wrapper around one loaded oracle library."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else load()

    # -- random draws -----------------------------------------------------
    def mix64(self, z: int) -> int:
        return int(self.lib.oracle_mix64(z))

    def draw(self, seed: int, b: int, n: int, i: int, t: int) -> int:
        return int(self.lib.oracle_draw(seed, b, n, i, t))

    # -- graph --------------------------------------------------------------
    def graph(self, n, radius, global_idx, num_random, num_graphs=1, causal=False, seed=0,
              layout=0):
        """Returns (row_ptr int64[num_graphs, n+1], list of col_idx int32 arrays).
        layout 0: seeded random extras; 1: evenly spaced extras."""
        g = np.ascontiguousarray(np.asarray(global_idx, dtype=np.int32))
        gp = _ptr(g) if g.size else None
        nnz = np.zeros(num_graphs, dtype=np.int64)
        args = (n, radius, g.size, gp, num_random, num_graphs, int(bool(causal)), seed,
                int(layout))
        _check(self.lib.oracle_graph_nnz_layout(*args, _ptr(nnz)), "oracle_graph_nnz")
        row_ptr = np.zeros((num_graphs, n + 1), dtype=np.int64)
        cols = np.zeros(max(int(nnz.sum()), 1), dtype=np.int32)
        _check(self.lib.oracle_graph_build_layout(*args, _ptr(row_ptr), _ptr(cols)),
               "oracle_graph_build")
        out, base = [], 0
        for gr in range(num_graphs):
            out.append(cols[base:base + int(nnz[gr])].copy())
            base += int(nnz[gr])
        return row_ptr, out

    def block_graph(self, n, block, local_blocks, num_random_blocks, num_global_blocks,
                    num_graphs=1, seed=0):
        """BigBird block graph ("1.2.1 Static sparsity", section 2, eq. 13 and
        the twelve-block example). The sequence splits into N = n / block
        blocks. Query block I < g_b (a global block) reads every key block;
        any other reads the local blocks I - h .. I + h (h = (c - 1) / 2,
        clipped to the sequence), the global blocks 0 .. g_b - 1, and s random
        blocks drawn from the rest: draw t of block I of graph b is
        SplitMix64's counter-based output at (b N + I, t) (the same generator
        as the token graph), mapped to a block by (u >> 32) N >> 32, kept if
        new; when at most s blocks remain, all of them are taken. Every token
        of a query block reads every token of its key blocks.

        Returns (row_ptr int64[graphs, n + 1], cols per graph, key blocks:
        per graph a list over query blocks of ascending block lists)."""
        if block < 1 or n % block != 0:
            raise OracleError("block graph: block must divide n")
        if local_blocks < 1 or local_blocks % 2 == 0:
            raise OracleError("block graph: local_blocks must be odd")
        N = n // block
        h = (local_blocks - 1) // 2
        gb, s = int(num_global_blocks), int(num_random_blocks)
        if gb < 0 or s < 0 or gb > N:
            raise OracleError("block graph: bad global or random block count")
        row_ptr = np.zeros((num_graphs, n + 1), dtype=np.int64)
        cols, blocks = [], []
        for gr in range(num_graphs):
            keys = []
            for I in range(N):
                if I < gb:
                    keys.append(list(range(N)))
                    continue
                base = set(range(max(0, I - h), min(N - 1, I + h) + 1)) | set(range(gb))
                pool = [J for J in range(N) if J not in base]
                if len(pool) <= s:
                    chosen = set(pool)
                else:
                    chosen, t = set(), 0
                    while len(chosen) < s:
                        if t >= (1 << 20):
                            raise OracleError("block graph: draw budget exhausted")
                        u = self.draw(seed, gr, N, I, t)
                        t += 1
                        J = ((u >> 32) * N) >> 32
                        if J not in base:
                            chosen.add(J)
                keys.append(sorted(base | chosen))
            row_cols = [np.concatenate([np.arange(J * block, (J + 1) * block, dtype=np.int32)
                                        for J in ks]) for ks in keys]
            deg = np.repeat([len(ks) * block for ks in keys], block)
            row_ptr[gr, 1:] = np.cumsum(deg)
            cols.append(np.concatenate([row_cols[i // block] for i in range(n)]).astype(np.int32))
            blocks.append(keys)
        return row_ptr, cols, blocks

    def dilated_graph(self, n, radius, dilation, global_idx):
        """Longformer's dilated window with global positions ("1.2.1 Static
        sparsity", section 1.2, eqs. 11 and 12): row i not in G reads
        {i + k delta : -r <= k <= r} within the sequence, plus G; a row in G
        reads every position. Returns (row_ptr int64[1, n + 1], [cols])."""
        if n < 1 or radius < 0 or dilation < 1:
            raise OracleError("dilated graph: bad arguments")
        G = sorted(set(int(x) for x in global_idx))
        if any(x < 0 or x >= n for x in G):
            raise OracleError("dilated graph: global position out of range")
        Gs = set(G)
        rows = []
        for i in range(n):
            if i in Gs:
                rows.append(np.arange(n, dtype=np.int32))
                continue
            s = {i + k * dilation for k in range(-radius, radius + 1)}
            s = {j for j in s if 0 <= j < n} | Gs
            rows.append(np.array(sorted(s), dtype=np.int32))
        row_ptr = np.zeros((1, n + 1), dtype=np.int64)
        row_ptr[0, 1:] = np.cumsum([len(r) for r in rows])
        return row_ptr, [np.concatenate(rows).astype(np.int32)]

    # -- per (batch, head) arithmetic ----------------------------------------
    def scores_softmax(self, Q, K, row_ptr, col_idx, threads=1):
        Q = np.ascontiguousarray(Q, dtype=np.float64)
        K = np.ascontiguousarray(K, dtype=np.float64)
        rp = np.ascontiguousarray(row_ptr, dtype=np.int64)
        ci = np.ascontiguousarray(col_idx, dtype=np.int32)
        n, d = Q.shape
        A = np.zeros(max(int(rp[-1]), 1), dtype=np.float64)
        _check(self.lib.oracle_scores_softmax(_ptr(Q), _ptr(K), n, d, _ptr(rp), _ptr(ci),
                                              _ptr(A), threads), "oracle_scores_softmax")
        return A[: int(rp[-1])]

    def scores(self, Q, K, row_ptr, col_idx, threads=1):
        Q = np.ascontiguousarray(Q, dtype=np.float64)
        K = np.ascontiguousarray(K, dtype=np.float64)
        rp = np.ascontiguousarray(row_ptr, dtype=np.int64)
        ci = np.ascontiguousarray(col_idx, dtype=np.int32)
        n, d = Q.shape
        S = np.zeros(max(int(rp[-1]), 1), dtype=np.float64)
        _check(self.lib.oracle_scores(_ptr(Q), _ptr(K), n, d, _ptr(rp), _ptr(ci), _ptr(S),
                                      threads), "oracle_scores")
        return S[: int(rp[-1])]

    def diffuse(self, A, V, row_ptr, col_idx, K_steps, alpha, threads=1):
        A = np.ascontiguousarray(A, dtype=np.float64)
        V = np.ascontiguousarray(V, dtype=np.float64)
        rp = np.ascontiguousarray(row_ptr, dtype=np.int64)
        ci = np.ascontiguousarray(col_idx, dtype=np.int32)
        n, d = V.shape
        if A.size == 0:
            A = np.zeros(1)
        Z = np.zeros_like(V)
        _check(self.lib.oracle_diffuse(_ptr(A), _ptr(V), n, d, _ptr(rp), _ptr(ci), K_steps,
                                       float(alpha), _ptr(Z), threads), "oracle_diffuse")
        return Z

    def diffuse_theta(self, A, V, row_ptr, col_idx, theta, threads=1):
        """Z = sum_k theta[k] A^k V, k = 0 .. len(theta) - 1."""
        A = np.ascontiguousarray(A, dtype=np.float64)
        V = np.ascontiguousarray(V, dtype=np.float64)
        th = np.ascontiguousarray(theta, dtype=np.float64)
        rp = np.ascontiguousarray(row_ptr, dtype=np.int64)
        ci = np.ascontiguousarray(col_idx, dtype=np.int32)
        n, d = V.shape
        if A.size == 0:
            A = np.zeros(1)
        Z = np.zeros_like(V)
        _check(self.lib.oracle_diffuse_theta(_ptr(A), _ptr(V), n, d, _ptr(rp), _ptr(ci),
                                             len(th) - 1, _ptr(th), _ptr(Z), threads),
               "oracle_diffuse_theta")
        return Z

    def attn_theta(self, Q, K, V, row_ptr, col_idx, theta, threads=1):
        """Whole path with general diffusion coefficients for one (batch, head)."""
        A = self.scores_softmax(Q, K, row_ptr, col_idx, threads)
        return self.diffuse_theta(A, V, row_ptr, col_idx, theta, threads)

    def attn_backward(self, Q, K, V, dZ, row_ptr, col_idx, K_steps, alpha):
        """(dQ, dK, dV): gradients of sum(dZ * attn(Q, K, V)) for one (batch, head)."""
        Q, K, V, dZ = (np.ascontiguousarray(x, dtype=np.float64) for x in (Q, K, V, dZ))
        rp = np.ascontiguousarray(row_ptr, dtype=np.int64)
        ci = np.ascontiguousarray(col_idx, dtype=np.int32)
        n, d = Q.shape
        dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
        _check(self.lib.oracle_attn_backward(_ptr(Q), _ptr(K), _ptr(V), _ptr(dZ), n, d, _ptr(rp),
                                             _ptr(ci), K_steps, float(alpha), _ptr(dQ), _ptr(dK),
                                             _ptr(dV)), "oracle_attn_backward")
        return dQ, dK, dV

    def layer_forward(self, X, W_qkv, W_o, H, row_ptr, cols, K_steps, alpha, round_bf16=False,
                      threads=1):
        """One layer around the path ("Diffuser" notes sections 2.1 and 2.4):
        [Q | K | V] = X W_qkv per head, Z per (b, h) by the whole path, Y =
        concat_h(Z) W_o. X: [B, n, d_model]; row_ptr: [graphs, n+1]; cols: per
        graph. round_bf16: Q, K, V and Z are held in bf16 (round to nearest
        even), as a bf16 implementation stores them."""
        X = np.asarray(X, dtype=np.float64)
        B, n, _ = X.shape
        d = W_qkv.shape[1] // (3 * H)
        T = X @ np.asarray(W_qkv, dtype=np.float64)            # [B, n, 3 H d]
        if round_bf16:
            T = round_bf16_rne(T)
        T = T.reshape(B, n, 3, H, d)
        Z = np.zeros((B, H, n, d))
        for b in range(B):
            gr = 0 if len(cols) == 1 else b
            for h in range(H):
                Z[b, h] = self.attn(T[b, :, 0, h], T[b, :, 1, h], T[b, :, 2, h], row_ptr[gr],
                                    cols[gr], K_steps, alpha, threads)
        if round_bf16:
            Z = round_bf16_rne(Z)
        Zc = Z.transpose(0, 2, 1, 3).reshape(B, n, H * d)
        return Zc @ np.asarray(W_o, dtype=np.float64)

    def attn(self, Q, K, V, row_ptr, col_idx, K_steps, alpha, threads=1):
        """Whole path for one (batch, head): scores, softmax, K diffusion steps."""
        A = self.scores_softmax(Q, K, row_ptr, col_idx, threads)
        return self.diffuse(A, V, row_ptr, col_idx, K_steps, alpha, threads)
