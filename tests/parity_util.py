"""Comparison helpers shared by the GPU parity tests.

Tolerances (on Z, against the double-precision oracle):
  fp32 storage: |z - z_ref| <= 1e-4 * max(|z_ref|, 1e-2)  (max relative error
                1e-4 with a 1e-2 floor on the denominator);
  bf16 storage: |z - z_ref| <= 2e-2 absolute for every (K, alpha). A and
                every Z_k are stored in bf16, so rounding errors of up to
                2^-8 relative enter at each step; with the row rescale c_i
                each step's matrix is row-stochastic, so those errors average
                out instead of compounding: at K = 10, alpha = 0 the worst
                case measured is 0.6 of the bound
                (test_bf16_long_diffusion_plain_bound).
Edge-softmax rows: |sum_j A_ij - 1| <= 1e-5 (fp32), <= 2^-8 + 1e-6 (bf16,
whose round-to-nearest-even step is at most 2^-8 relative per weight).
"""
from __future__ import annotations

import os

import numpy as np

F32_REL = 1e-4
F32_FLOOR = 1e-2
BF16_ABS = 2e-2
ROWSUM_F32 = 1e-5
ROWSUM_BF16 = 2.0 ** -8 + 1e-6


def oracle_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def bf16_tolerance(K: int = 5, alpha: float = 0.1) -> float:
    """The bf16 bound; the same for every (K, alpha)."""
    return BF16_ABS


def z_error(got: np.ndarray, ref: np.ndarray, dtype: str, K: int = 5, alpha: float = 0.1) -> float:
    """Error in units of the tolerance (<= 1 passes)."""
    d = np.abs(got.astype(np.float64) - ref)
    if dtype == "f32":
        return float((d / (F32_REL * np.maximum(np.abs(ref), F32_FLOOR))).max(initial=0.0))
    return float(d.max(initial=0.0) / bf16_tolerance(K, alpha))


def assert_z_close(got, ref, dtype, what="", K: int = 5, alpha: float = 0.1):
    e = z_error(got, ref, dtype, K, alpha)
    assert e <= 1.0, f"{what}: error {e:.3f} x tolerance ({dtype})"
    return e


def rowsum_bound(dtype: str) -> float:
    return ROWSUM_F32 if dtype == "f32" else ROWSUM_BF16


def dtype_name(t) -> str:
    import torch
    return "f32" if t == torch.float32 else "bf16"


def slot_permutation(slot_row, slot_col, row_ptr, col_idx):
    """Indices of the non-padding weight slots in ascending-CSR order.

    Checks that padding slots carry row and column -1 and that the other
    slots hold exactly the graph's edges, each once, so A in slot layout maps
    one-to-one onto the edges."""
    slot_row = np.asarray(slot_row)
    slot_col = np.asarray(slot_col)
    n = len(row_ptr) - 1
    valid = slot_col >= 0
    assert np.array_equal(valid, slot_row >= 0), "padding slots carry row and column -1"
    idx = np.nonzero(valid)[0]
    order = np.lexsort((slot_col[idx], slot_row[idx]))
    perm = idx[order]
    assert np.array_equal(slot_row[perm], np.repeat(np.arange(n), np.diff(row_ptr))), "slot rows"
    assert np.array_equal(slot_col[perm], col_idx), "slot columns"
    return perm, ~valid
