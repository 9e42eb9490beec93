"""MI355X (gfx950) Diffuser attention-diffusion path: Python binding.

Argument marshalling only: every step of the path runs in the HIP library
``libdiffuser.so`` (C ABI declared in ``include/diffuser.h``), reached through
ctypes. PyTorch supplies device memory and the current stream. There is no
fallback: if the library is missing, every call raises.

Functions mirror the C ABI names:
  build_graph     -> diffuser_build_graph (diffuser_build_graph_layout with layout=)
  graph_from_csr  -> diffuser_graph_from_csr
  workspace_size  -> diffuser_attn_workspace_size
  attn            -> diffuser_attn
  scores_softmax  -> diffuser_scores_softmax
  diffuse         -> diffuser_diffuse
  diffuse_workspace_size -> diffuser_diffuse_workspace_size
  diffuse_noalloc -> diffuser_diffuse_noalloc
  attn_backward   -> diffuser_attn_backward (+ _workspace_size)
  layer_forward   -> diffuser_layer_forward (+ _workspace_size)
  attn_theta      -> diffuser_attn_theta
  diffuse_theta   -> diffuser_diffuse_theta
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdiffuser.so")

F32, BF16 = 0, 1

STATUS_NAMES = {
    0: "DIFFUSER_OK", 1: "DIFFUSER_ERR_INVALID_ARG", 2: "DIFFUSER_ERR_UNSUPPORTED",
    3: "DIFFUSER_ERR_OUT_OF_MEMORY", 4: "DIFFUSER_ERR_HIP", 5: "DIFFUSER_ERR_INTERNAL",
}

# Every symbol the header declares.
ABI_SYMBOLS = (
    "diffuser_build_graph", "diffuser_build_graph_layout", "diffuser_graph_from_csr",
    "diffuser_build_block_graph", "diffuser_build_dilated_graph",
    "diffuser_graph_info",
    "diffuser_graph_copy_csr", "diffuser_graph_copy_slots", "diffuser_graph_destroy",
    "diffuser_attn_workspace_size",
    "diffuser_attn", "diffuser_scores_softmax", "diffuser_diffuse",
    "diffuser_diffuse_workspace_size", "diffuser_diffuse_noalloc",
    "diffuser_attn_theta", "diffuser_diffuse_theta",
    "diffuser_csr_workspace_size", "diffuser_scores_softmax_csr", "diffuser_diffuse_csr",
    "diffuser_attn_backward_workspace_size", "diffuser_attn_backward",
    "diffuser_layer_workspace_size", "diffuser_layer_forward",
    "diffuser_status_string", "diffuser_last_error",
)


class DiffuserError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


class _BlockGraphDesc(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int64),
        ("block", ctypes.c_int32),
        ("local_blocks", ctypes.c_int32),
        ("num_random_blocks", ctypes.c_int32),
        ("num_global_blocks", ctypes.c_int32),
        ("num_graphs", ctypes.c_int32),
        ("seed", ctypes.c_uint64),
    ]


class _GraphDesc(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int64),
        ("window_radius", ctypes.c_int32),
        ("num_global", ctypes.c_int32),
        ("global_idx", ctypes.c_void_p),
        ("num_random", ctypes.c_int32),
        ("num_graphs", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("seed", ctypes.c_uint64),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Loads libdiffuser.so; raises if it has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is missing: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    i32, i64, u64, p, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_size_t
    st = ctypes.c_int
    lib.diffuser_build_graph.argtypes = [ctypes.POINTER(_GraphDesc), p, ctypes.POINTER(p)]
    lib.diffuser_build_graph.restype = st
    lib.diffuser_build_graph_layout.argtypes = [ctypes.POINTER(_GraphDesc), i32, p,
                                                ctypes.POINTER(p)]
    lib.diffuser_build_graph_layout.restype = st
    lib.diffuser_graph_from_csr.argtypes = [i64, i32, p, p, p, ctypes.POINTER(p)]
    lib.diffuser_build_block_graph.argtypes = [ctypes.POINTER(_BlockGraphDesc), p,
                                               ctypes.POINTER(p)]
    lib.diffuser_build_block_graph.restype = st
    lib.diffuser_build_dilated_graph.argtypes = [i64, i32, i32, i32, p, p, ctypes.POINTER(p)]
    lib.diffuser_build_dilated_graph.restype = st
    lib.diffuser_graph_from_csr.restype = st
    lib.diffuser_graph_info.argtypes = [p, p, p, p, p]
    lib.diffuser_graph_info.restype = st
    lib.diffuser_graph_copy_csr.argtypes = [p, i32, p, p, p]
    lib.diffuser_graph_copy_csr.restype = st
    lib.diffuser_graph_copy_slots.argtypes = [p, i32, p, p, p]
    lib.diffuser_graph_copy_slots.restype = st
    lib.diffuser_graph_destroy.argtypes = [p]
    lib.diffuser_graph_destroy.restype = None
    lib.diffuser_attn_workspace_size.argtypes = [p, i32, i32, i32, i32, st, ctypes.POINTER(sz)]
    lib.diffuser_attn_workspace_size.restype = st
    lib.diffuser_diffuse_workspace_size.argtypes = [p, i32, i32, i32, i32, st,
                                                    ctypes.POINTER(sz)]
    lib.diffuser_diffuse_workspace_size.restype = st
    lib.diffuser_diffuse_noalloc.argtypes = [p, p, st, i32, i32, i32, p, i32, ctypes.c_float, p, p]
    lib.diffuser_diffuse_noalloc.restype = st
    lib.diffuser_attn.argtypes = [p, p, p, st, i32, i32, i32, i32, p, i32, ctypes.c_float, p, p,
                                  sz, p]
    lib.diffuser_attn.restype = st
    lib.diffuser_scores_softmax.argtypes = [p, p, st, i32, i32, i32, p, p, p, sz, p]
    lib.diffuser_scores_softmax.restype = st
    lib.diffuser_diffuse.argtypes = [p, p, st, i32, i32, i32, p, i32, ctypes.c_float, p, p, sz, p]
    lib.diffuser_diffuse.restype = st
    lib.diffuser_csr_workspace_size.argtypes = [p, i32, i32, i32, i32, st, ctypes.POINTER(sz)]
    lib.diffuser_csr_workspace_size.restype = st
    lib.diffuser_scores_softmax_csr.argtypes = [p, p, st, i32, i32, i32, p, p, p, sz, p]
    lib.diffuser_scores_softmax_csr.restype = st
    lib.diffuser_diffuse_csr.argtypes = [p, p, st, i32, i32, i32, p, i32, ctypes.c_float, p, p,
                                         sz, p]
    lib.diffuser_diffuse_csr.restype = st
    lib.diffuser_attn_backward_workspace_size.argtypes = [p, i32, i32, i32, i32, st,
                                                          ctypes.POINTER(sz)]
    lib.diffuser_attn_backward_workspace_size.restype = st
    lib.diffuser_attn_backward.argtypes = [p, p, p, p, st, i32, i32, i32, p, i32, ctypes.c_float,
                                           p, p, p, p, sz, p]
    lib.diffuser_attn_backward.restype = st
    lib.diffuser_layer_workspace_size.argtypes = [p, i32, i32, i32, i32, st, ctypes.POINTER(sz)]
    lib.diffuser_layer_workspace_size.restype = st
    lib.diffuser_layer_forward.argtypes = [p, p, p, st, i32, i32, i32, i32, p, i32,
                                           ctypes.c_float, p, p, sz, p]
    lib.diffuser_layer_forward.restype = st
    lib.diffuser_attn_theta.argtypes = [p, p, p, st, i32, i32, i32, i32, p, i32, p, p, p, sz, p]
    lib.diffuser_attn_theta.restype = st
    lib.diffuser_diffuse_theta.argtypes = [p, p, st, i32, i32, i32, p, i32, p, p, p, sz, p]
    lib.diffuser_diffuse_theta.restype = st
    lib.diffuser_status_string.argtypes = [st]
    lib.diffuser_status_string.restype = ctypes.c_char_p
    lib.diffuser_last_error.argtypes = []
    lib.diffuser_last_error.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load_library().diffuser_last_error().decode(errors="replace")
        raise DiffuserError(status, msg)


def _torch():
    import torch
    return torch


def _stream_handle(device=None) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t) -> int:
    torch = _torch()
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    raise DiffuserError(2, f"dtype {t} is not supported (float32 or bfloat16)")


class Graph:
    """Owns a diffuser_graph handle; freed with diffuser_graph_destroy."""

    def __init__(self, handle: int, desc: Optional[dict] = None):
        self._lib = load_library()
        self.handle = ctypes.c_void_p(handle)
        n = ctypes.c_int64()
        ng = ctypes.c_int32()
        _check(self._lib.diffuser_graph_info(self.handle, ctypes.byref(n), ctypes.byref(ng), None,
                                             None))
        self.n, self.num_graphs = int(n.value), int(ng.value)
        nnz = np.zeros(self.num_graphs, dtype=np.int64)
        slots = np.zeros(self.num_graphs, dtype=np.int64)
        _check(self._lib.diffuser_graph_info(self.handle, None, None,
                                             nnz.ctypes.data_as(ctypes.c_void_p),
                                             slots.ctypes.data_as(ctypes.c_void_p)))
        self.nnz = [int(x) for x in nnz]
        self.slots = [int(x) for x in slots]
        self.desc = desc

    def copy_csr(self, graph: int = 0):
        """(row_ptr int64[n+1], col_idx int32[nnz]) of one graph, on the host."""
        rp = np.zeros(self.n + 1, dtype=np.int64)
        ci = np.zeros(max(self.nnz[graph], 1), dtype=np.int32)
        _check(self._lib.diffuser_graph_copy_csr(self.handle, graph,
                                                 rp.ctypes.data_as(ctypes.c_void_p),
                                                 ci.ctypes.data_as(ctypes.c_void_p),
                                                 ctypes.c_void_p(_stream_handle())))
        return rp, ci[: self.nnz[graph]]

    def copy_slots(self, graph: int = 0):
        """(slot_row int32[slots], slot_col int32[slots]) of one graph: slot s
        of A's (b, h) block holds the weight of edge (slot_row[s],
        slot_col[s]); -1 marks padding."""
        sr = np.zeros(max(self.slots[graph], 1), dtype=np.int32)
        sc = np.zeros(max(self.slots[graph], 1), dtype=np.int32)
        _check(self._lib.diffuser_graph_copy_slots(self.handle, graph,
                                                   sr.ctypes.data_as(ctypes.c_void_p),
                                                   sc.ctypes.data_as(ctypes.c_void_p),
                                                   ctypes.c_void_p(_stream_handle())))
        return sr[: self.slots[graph]], sc[: self.slots[graph]]

    def edges(self, B: int, H: int) -> int:
        """Edges summed over every (b, h) pair (padding slots excluded)."""
        if self.num_graphs == 1:
            return B * H * self.nnz[0]
        return H * sum(self.nnz)

    def a_numel(self, B: int, H: int) -> int:
        if self.num_graphs == 1:
            return B * H * self.slots[0]
        return H * sum(self.slots)

    def a_offset(self, b: int, h: int, H: int) -> int:
        """Start of the (b, h) block inside the A layout."""
        if self.num_graphs == 1:
            return (b * H + h) * self.slots[0]
        return H * sum(self.slots[:b]) + h * self.slots[b]

    def close(self):
        if self.handle is not None and self.handle.value:
            self._lib.diffuser_graph_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


EXTRAS_RANDOM = 0   # seeded uniform draws
EXTRAS_EVEN = 1     # evenly spaced over each row's pool


def build_graph(n: int, radius: int, global_idx: Sequence[int], num_random: int,
                num_graphs: int = 1, causal: bool = False, seed: int = 0,
                layout: int = EXTRAS_RANDOM) -> Graph:
    """diffuser_build_graph (layout EXTRAS_RANDOM) or
    diffuser_build_graph_layout."""
    lib = load_library()
    g = np.ascontiguousarray(np.asarray(list(global_idx), dtype=np.int32))
    desc = _GraphDesc(n, radius, g.size, g.ctypes.data if g.size else None, num_random,
                      num_graphs, int(bool(causal)), seed)
    out = ctypes.c_void_p()
    if layout == EXTRAS_RANDOM:
        _check(lib.diffuser_build_graph(ctypes.byref(desc), ctypes.c_void_p(_stream_handle()),
                                        ctypes.byref(out)))
    else:
        _check(lib.diffuser_build_graph_layout(ctypes.byref(desc), int(layout),
                                               ctypes.c_void_p(_stream_handle()),
                                               ctypes.byref(out)))
    return Graph(out.value, dict(n=n, radius=radius, global_idx=tuple(g.tolist()),
                                 num_random=num_random, num_graphs=num_graphs,
                                 causal=bool(causal), seed=seed, layout=int(layout)))


def graph_from_csr(n: int, row_ptr, col_idx) -> Graph:
    """row_ptr: int64 [num_graphs, n+1] (each from 0); col_idx: the graphs'
    columns concatenated (or a list of per-graph arrays)."""
    lib = load_library()
    rp = np.ascontiguousarray(np.atleast_2d(np.asarray(row_ptr, dtype=np.int64)))
    if isinstance(col_idx, (list, tuple)):
        col_idx = np.concatenate([np.asarray(c, dtype=np.int32) for c in col_idx]) \
            if len(col_idx) else np.zeros(0, np.int32)
    ci = np.ascontiguousarray(np.asarray(col_idx, dtype=np.int32))
    out = ctypes.c_void_p()
    _check(lib.diffuser_graph_from_csr(n, rp.shape[0], rp.ctypes.data_as(ctypes.c_void_p),
                                       ci.ctypes.data_as(ctypes.c_void_p) if ci.size else None,
                                       ctypes.c_void_p(_stream_handle()), ctypes.byref(out)))
    return Graph(out.value)


def build_block_graph(n: int, block: int, local_blocks: int, num_random_blocks: int,
                      num_global_blocks: int, num_graphs: int = 1, seed: int = 0) -> Graph:
    """diffuser_build_block_graph: the BigBird block layout."""
    lib = load_library()
    desc = _BlockGraphDesc(n, block, local_blocks, num_random_blocks, num_global_blocks,
                           num_graphs, seed)
    out = ctypes.c_void_p()
    _check(lib.diffuser_build_block_graph(ctypes.byref(desc), ctypes.c_void_p(_stream_handle()),
                                          ctypes.byref(out)))
    return Graph(out.value, dict(n=n, block=block, local_blocks=local_blocks,
                                 num_random_blocks=num_random_blocks,
                                 num_global_blocks=num_global_blocks, num_graphs=num_graphs,
                                 seed=seed))


def build_dilated_graph(n: int, radius: int, dilation: int, global_idx: Sequence[int]) -> Graph:
    """diffuser_build_dilated_graph: Longformer's dilated window with globals."""
    lib = load_library()
    g = np.ascontiguousarray(np.asarray(list(global_idx), dtype=np.int32))
    out = ctypes.c_void_p()
    _check(lib.diffuser_build_dilated_graph(n, radius, dilation, g.size,
                                            g.ctypes.data_as(ctypes.c_void_p) if g.size else None,
                                            ctypes.c_void_p(_stream_handle()),
                                            ctypes.byref(out)))
    return Graph(out.value, dict(n=n, radius=radius, dilation=dilation,
                                 global_idx=tuple(g.tolist())))


def workspace_size(graph: Graph, B: int, H: int, d_h: int, d_v: int, dtype) -> int:
    lib = load_library()
    out = ctypes.c_size_t()
    _check(lib.diffuser_attn_workspace_size(graph.handle, B, H, d_h, d_v, _dtype_code(dtype),
                                            ctypes.byref(out)))
    return int(out.value)


def diffuse_workspace_size(graph: Graph, B: int, H: int, d_v: int, K: int, dtype) -> int:
    """Workspace bytes of diffuse / diffuse_theta with K steps (0: none)."""
    lib = load_library()
    out = ctypes.c_size_t()
    _check(lib.diffuser_diffuse_workspace_size(graph.handle, B, H, d_v, K, _dtype_code(dtype),
                                               ctypes.byref(out)))
    return int(out.value)


def _diffuse_workspace(graph, v, K, workspace):
    if workspace is None:
        B, H, _, d_v = v.shape
        need = diffuse_workspace_size(graph, B, H, d_v, K, v.dtype)
        workspace = _torch().empty(max(need, 1), dtype=_torch().uint8, device=v.device)
    return workspace


def _check_bhnd(t, name, n):
    if not t.is_cuda or not t.is_contiguous() or t.dim() != 4 or t.shape[2] != n:
        raise DiffuserError(1, f"{name} must be a contiguous CUDA tensor [B, H, n={n}, d]")


def _workspace(graph, B, H, d_h, d_v, dtype, device, workspace):
    torch = _torch()
    need = workspace_size(graph, B, H, d_h, d_v, dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return workspace, need


def attn(q, k, v, graph: Graph, K: int, alpha: float, out=None, workspace=None):
    """Z = K diffusion steps of the edge-softmax attention of (q, k) over v."""
    torch = _torch()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _check_bhnd(t, nm, graph.n)
    B, H, _, d_h = q.shape
    d_v = v.shape[3]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or not (q.dtype == k.dtype == v.dtype):
        raise DiffuserError(1, "q, k, v shapes/dtypes disagree")
    if out is None:
        out = torch.empty_like(v)
    workspace, _ = _workspace(graph, B, H, d_h, d_v, q.dtype, q.device, workspace)
    lib = load_library()
    _check(lib.diffuser_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q.dtype), B, H,
                             d_h, d_v, graph.handle, K, float(alpha), out.data_ptr(),
                             workspace.data_ptr(), workspace.numel(),
                             ctypes.c_void_p(_stream_handle(q.device))))
    return out


def scores_softmax(q, k, graph: Graph, out=None):
    """Edge-softmax weights A (1-D, the (b, h)-blocked CSR layout)."""
    torch = _torch()
    for t, nm in ((q, "q"), (k, "k")):
        _check_bhnd(t, nm, graph.n)
    B, H, _, d_h = q.shape
    if k.shape != q.shape or q.dtype != k.dtype:
        raise DiffuserError(1, "q, k shapes/dtypes disagree")
    if out is None:
        out = torch.empty(graph.a_numel(B, H), dtype=q.dtype, device=q.device)
    lib = load_library()
    _check(lib.diffuser_scores_softmax(q.data_ptr(), k.data_ptr(), _dtype_code(q.dtype), B, H, d_h,
                                       graph.handle, out.data_ptr(), None, 0,
                                       ctypes.c_void_p(_stream_handle(q.device))))
    return out


def diffuse(A, v, graph: Graph, K: int, alpha: float, out=None, workspace=None):
    """K steps of Z <- (1 - alpha) A Z + alpha V from Z = V with given A."""
    torch = _torch()
    _check_bhnd(v, "v", graph.n)
    B, H, _, d_v = v.shape
    if not A.is_cuda or not A.is_contiguous() or A.dtype != v.dtype or \
            A.numel() != graph.a_numel(B, H):
        raise DiffuserError(1, "A must be a contiguous CUDA tensor in the A layout")
    if out is None:
        out = torch.empty_like(v)
    workspace = _diffuse_workspace(graph, v, K, workspace)
    lib = load_library()
    _check(lib.diffuser_diffuse(A.data_ptr(), v.data_ptr(), _dtype_code(v.dtype), B, H, d_v,
                                graph.handle, K, float(alpha), out.data_ptr(),
                                workspace.data_ptr(), workspace.numel(),
                                ctypes.c_void_p(_stream_handle(v.device))))
    return out


def diffuse_noalloc(A, v, graph: Graph, K: int, alpha: float, out):
    """diffuse() through the entry point that allocates nothing: its scratch
    is a fixed device array inside the library (64 MiB per GPU); out must be
    given."""
    _check_bhnd(v, "v", graph.n)
    _check_bhnd(out, "out", graph.n)
    B, H, _, d_v = v.shape
    if not A.is_cuda or not A.is_contiguous() or A.dtype != v.dtype or \
            A.numel() != graph.a_numel(B, H) or out.shape != v.shape or out.dtype != v.dtype:
        raise DiffuserError(1, "A, v and out must match the A layout and each other")
    lib = load_library()
    _check(lib.diffuser_diffuse_noalloc(A.data_ptr(), v.data_ptr(), _dtype_code(v.dtype), B, H,
                                        d_v, graph.handle, K, float(alpha), out.data_ptr(),
                                        ctypes.c_void_p(_stream_handle(v.device))))
    return out


def csr_workspace_size(graph: Graph, B: int, H: int, d: int, K: int, dtype) -> int:
    """Workspace bytes accepted by scores_softmax_csr and diffuse_csr."""
    lib = load_library()
    out = ctypes.c_size_t()
    _check(lib.diffuser_csr_workspace_size(graph.handle, B, H, d, K, _dtype_code(dtype),
                                           ctypes.byref(out)))
    return int(out.value)


def _csr_workspace(graph, B, H, d, K, dtype, device, workspace):
    if workspace is None:
        need = csr_workspace_size(graph, B, H, d, K, dtype)
        workspace = _torch().empty(max(need, 1), dtype=_torch().uint8, device=device)
    return workspace


def scores_softmax_csr(q, k, graph: Graph, out=None, workspace=None):
    """Edge-softmax weights in CSR order (1-D, (b, h) blocks of nnz each)."""
    torch = _torch()
    for t, nm in ((q, "q"), (k, "k")):
        _check_bhnd(t, nm, graph.n)
    B, H, _, d_h = q.shape
    if k.shape != q.shape or q.dtype != k.dtype:
        raise DiffuserError(1, "q, k shapes/dtypes disagree")
    if out is None:
        out = torch.empty(graph.edges(B, H), dtype=q.dtype, device=q.device)
    elif not out.is_cuda or not out.is_contiguous() or out.dtype != q.dtype or \
            out.numel() != graph.edges(B, H):
        raise DiffuserError(1, "out must be a contiguous CUDA tensor of the edges in CSR order")
    workspace = _csr_workspace(graph, B, H, d_h, 0, q.dtype, q.device, workspace)
    lib = load_library()
    _check(lib.diffuser_scores_softmax_csr(q.data_ptr(), k.data_ptr(), _dtype_code(q.dtype), B,
                                           H, d_h, graph.handle, out.data_ptr(),
                                           workspace.data_ptr(), workspace.numel(),
                                           ctypes.c_void_p(_stream_handle(q.device))))
    return out


def diffuse_csr(A_csr, v, graph: Graph, K: int, alpha: float, out=None, workspace=None):
    """diffuse() with the weights given in CSR order."""
    torch = _torch()
    _check_bhnd(v, "v", graph.n)
    B, H, _, d_v = v.shape
    if not A_csr.is_cuda or not A_csr.is_contiguous() or A_csr.dtype != v.dtype or \
            A_csr.numel() != graph.edges(B, H):
        raise DiffuserError(1, "A_csr must be a contiguous CUDA tensor of the edges in CSR order")
    if out is None:
        out = torch.empty_like(v)
    workspace = _csr_workspace(graph, B, H, d_v, K, v.dtype, v.device, workspace)
    lib = load_library()
    _check(lib.diffuser_diffuse_csr(A_csr.data_ptr(), v.data_ptr(), _dtype_code(v.dtype), B, H,
                                    d_v, graph.handle, K, float(alpha), out.data_ptr(),
                                    workspace.data_ptr(), workspace.numel(),
                                    ctypes.c_void_p(_stream_handle(v.device))))
    return out


def _theta_array(theta):
    th = [float(x) for x in theta]
    if len(th) < 1:
        raise DiffuserError(1, "theta needs at least one coefficient")
    return (ctypes.c_float * len(th))(*th), len(th) - 1


def attn_theta(q, k, v, graph: Graph, theta, out=None, workspace=None):
    """Z = sum_k theta[k] A^k V with A the edge-softmax weights of (q, k)."""
    torch = _torch()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _check_bhnd(t, nm, graph.n)
    B, H, _, d_h = q.shape
    d_v = v.shape[3]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or not (q.dtype == k.dtype == v.dtype):
        raise DiffuserError(1, "q, k, v shapes/dtypes disagree")
    if out is None:
        out = torch.empty_like(v)
    workspace, _ = _workspace(graph, B, H, d_h, d_v, q.dtype, q.device, workspace)
    th, K = _theta_array(theta)
    lib = load_library()
    _check(lib.diffuser_attn_theta(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q.dtype),
                                   B, H, d_h, d_v, graph.handle, K, th, out.data_ptr(),
                                   workspace.data_ptr(), workspace.numel(),
                                   ctypes.c_void_p(_stream_handle(q.device))))
    return out


def diffuse_theta(A, v, graph: Graph, theta, out=None, workspace=None):
    """Z = sum_k theta[k] A^k V with given A."""
    torch = _torch()
    _check_bhnd(v, "v", graph.n)
    B, H, _, d_v = v.shape
    if not A.is_cuda or not A.is_contiguous() or A.dtype != v.dtype or \
            A.numel() != graph.a_numel(B, H):
        raise DiffuserError(1, "A must be a contiguous CUDA tensor in the A layout")
    if out is None:
        out = torch.empty_like(v)
    th, K = _theta_array(theta)
    workspace = _diffuse_workspace(graph, v, K, workspace)
    lib = load_library()
    _check(lib.diffuser_diffuse_theta(A.data_ptr(), v.data_ptr(), _dtype_code(v.dtype), B, H, d_v,
                                      graph.handle, K, th, out.data_ptr(), workspace.data_ptr(),
                                      workspace.numel(), ctypes.c_void_p(_stream_handle(v.device))))
    return out


def attn_backward(q, k, v, dz, graph: Graph, K: int, alpha: float, workspace=None):
    """(dq, dk, dv): gradients through attn(q, k, v, graph, K, alpha) of a loss
    whose gradient with respect to its output is dz."""
    torch = _torch()
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (dz, "dz")):
        _check_bhnd(t, nm, graph.n)
    if not (q.shape == k.shape == v.shape == dz.shape) or \
            not (q.dtype == k.dtype == v.dtype == dz.dtype):
        raise DiffuserError(1, "q, k, v, dz shapes/dtypes disagree")
    B, H, _, d = q.shape
    lib = load_library()
    need = ctypes.c_size_t()
    _check(lib.diffuser_attn_backward_workspace_size(graph.handle, B, H, d, K,
                                                     _dtype_code(q.dtype), ctypes.byref(need)))
    if workspace is None:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _check(lib.diffuser_attn_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), dz.data_ptr(),
                                      _dtype_code(q.dtype), B, H, d, graph.handle, K,
                                      float(alpha), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                      workspace.data_ptr(), workspace.numel(),
                                      ctypes.c_void_p(_stream_handle(q.device))))
    return dq, dk, dv


def layer_forward(x, w_qkv, w_o, graph: Graph, H: int, K: int, alpha: float, workspace=None):
    """Y = concat_h(attn(Q, K, V)) w_o with [Q | K | V] = x w_qkv per head.
    x: [B, n, d_model]; w_qkv: [d_model, 3 H d]; w_o: [H d, d_model]."""
    torch = _torch()
    if x.dim() != 3 or x.shape[1] != graph.n or not x.is_cuda or not x.is_contiguous():
        raise DiffuserError(1, "x must be a contiguous CUDA tensor [B, n, d_model]")
    B, _, d_model = x.shape
    if w_qkv.dim() != 2 or w_qkv.shape[0] != d_model or w_qkv.shape[1] % (3 * H):
        raise DiffuserError(1, "w_qkv must be [d_model, 3 H d]")
    d = w_qkv.shape[1] // (3 * H)
    if tuple(w_o.shape) != (H * d, d_model):
        raise DiffuserError(1, "w_o must be [H d, d_model]")
    for t in (w_qkv, w_o):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != x.dtype:
            raise DiffuserError(1, "weights must be contiguous CUDA tensors of x's dtype")
    lib = load_library()
    need = ctypes.c_size_t()
    _check(lib.diffuser_layer_workspace_size(graph.handle, B, H, d, d_model, _dtype_code(x.dtype),
                                             ctypes.byref(need)))
    if workspace is None:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=x.device)
    y = torch.empty_like(x)
    _check(lib.diffuser_layer_forward(x.data_ptr(), w_qkv.data_ptr(), w_o.data_ptr(),
                                      _dtype_code(x.dtype), B, H, d, d_model, graph.handle, K,
                                      float(alpha), y.data_ptr(), workspace.data_ptr(),
                                      workspace.numel(), ctypes.c_void_p(_stream_handle(x.device))))
    return y
