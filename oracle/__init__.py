"""Diffuser CPU oracle -- TEST INFRASTRUCTURE ONLY.

Plain double-precision CPU implementation of the Diffuser attention-diffusion
path (graph, edge scores, edge softmax, K-step personalized-PageRank
diffusion), written in C (``oracle.c``) and reached through ctypes.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module. It shares no code with the HIP library.

Sources: "Diffuser" reading notes sections 2.1 (eqs. S.1-S.5), 2.2, 2.4
(eq. S.7), 2.5; "1.2.1 Static sparsity" sections 1, 1.1 (eq. 5), 1.2 (eq. 12);
"038 BigBird" section 2 (union neighbourhood).
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
