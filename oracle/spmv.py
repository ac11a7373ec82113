"""Emulated sparse matrix-vector product y = A x, A in CSR, by the Ozaki scheme II
arithmetic of the dense path, written out on the CPU (oracle).

Test infrastructure only (see the package docstring).  [TME4], abstract: sparse
matrix-vector products are among the memory-bound kernels whose emulation pays the
per-input deconstruction term; the page names the workload, not how its scaling is
set.  Readings taken here (the plainest ones the dense path supports):

* Each row of A is a dot product of at most kmax terms, kmax = the caller's bound on
  the nonzeros of a row, so the bit budget is that of inner dimension kmax:
  (P_A, P_B) = scaling_bits(r, kmax); rows of A are scaled by the max rule over their
  nonzeros, x (a single column) by one exponent over all of its entries.
* An empty row gives +0.  A row holding Inf or NaN, a row longer than kmax and a row
  with a column index outside [0, cols) give NaN (the GPU path marks the same rows and
  never reads through a bad index); Inf or NaN in x makes every y NaN.
* Everything else is the dense reading: a' = RNE(2^e a), symmetric residues, exact
  integer row sums per modulus, CRT lift, y_i = RN(X_i 2^-(e_i + f)).
"""
from __future__ import annotations

import math

import numpy as np

from . import ozaki2, rns

NONFINITE = ozaki2.NONFINITE


def row_exponents(row_ptr: np.ndarray, vals: np.ndarray, p_a: int) -> np.ndarray:
    """Max-rule exponent of every CSR row: 2^(P_A-1) <= max |a| 2^e < 2^P_A over the
    row's nonzeros; 0 for an empty or all-zero row, NONFINITE for a row with Inf/NaN."""
    rows = len(row_ptr) - 1
    out = np.zeros(rows, dtype=np.int64)
    for i in range(rows):
        seg = np.asarray(vals[row_ptr[i]:row_ptr[i + 1]], dtype=np.float64)
        if seg.size:
            out[i] = ozaki2.scale_exponents(seg[None, :], p_a, 0)[0]
    return out


def bad_rows(row_ptr: np.ndarray, col_idx: np.ndarray, cols: int, kmax: int) -> np.ndarray:
    """Rows longer than kmax or holding a column index outside [0, cols)."""
    rows = len(row_ptr) - 1
    bad = np.zeros(rows, dtype=bool)
    for i in range(rows):
        c = np.asarray(col_idx[row_ptr[i]:row_ptr[i + 1]])
        bad[i] = c.size > kmax or bool(np.any((c < 0) | (c >= cols)))
    return bad


def spmv_csr(row_ptr, col_idx, vals, x, r: int, kmax: int, rows=None) -> np.ndarray:
    """Emulated y = A x (optionally only the listed rows).  x's exponent always comes
    from the whole of x, so a sampled row equals the same row of the full result."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col_idx = np.asarray(col_idx, dtype=np.int64)
    vals = np.asarray(vals, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    cols = x.shape[0]
    p_a, p_b = rns.scaling_bits(r, kmax)
    sel = np.arange(len(row_ptr) - 1) if rows is None else np.asarray(rows, dtype=np.int64)
    # the selected rows as their own CSR matrix
    starts, ends = row_ptr[sel], row_ptr[sel + 1]
    sub_ptr = np.concatenate([[0], np.cumsum(ends - starts)])
    take = np.concatenate([np.arange(s, e) for s, e in zip(starts, ends)]) if len(sel) else \
        np.zeros(0, dtype=np.int64)
    sub_vals, sub_cols = vals[take], col_idx[take]
    bad = bad_rows(sub_ptr, sub_cols, cols, kmax)
    e = row_exponents(sub_ptr, sub_vals, p_a)
    e = np.where(bad, NONFINITE, e)
    f = ozaki2.scale_exponents(x[:, None], p_b, 1)          # one exponent for x
    # residues: every nonzero with its row's exponent, x with its exponent
    row_of = np.repeat(np.arange(len(sel)), np.diff(sub_ptr))
    planes_a = ozaki2.residue_planes(sub_vals[:, None], e[row_of], r, 0)[:, :, 0]
    planes_x = ozaki2.residue_planes(x[:, None], f, r, 1)[:, 0, :]
    safe_cols = np.clip(sub_cols, 0, max(cols - 1, 0))
    prods = np.zeros((r, 1, len(sel)), dtype=np.int64)
    for l in range(r):
        terms = planes_a[l].astype(np.int64) * planes_x[l][safe_cols].astype(np.int64)
        prods[l, 0] = np.bincount(row_of, weights=terms, minlength=len(sel)).astype(np.int64)
    y = ozaki2.reconstruct(prods, r, f, e)[0]
    y[bad] = math.nan
    return y


def spmv_exact_definition(row_ptr, col_idx, vals, x, r: int, kmax: int) -> np.ndarray:
    """The plain definition for tiny inputs: y_i = RN(2^-(e_i+f) sum_p a'_p x'_col(p))
    with the scaled integers and the sum in Python integers (no residues, no CRT)."""
    row_ptr = [int(v) for v in row_ptr]
    x = np.asarray(x, dtype=np.float64)
    cols = x.shape[0]
    p_a, p_b = rns.scaling_bits(r, kmax)
    f = int(ozaki2.scale_exponents(x[:, None], p_b, 1)[0])
    e = row_exponents(np.asarray(row_ptr), np.asarray(vals, dtype=np.float64), p_a)
    bad = bad_rows(np.asarray(row_ptr), np.asarray(col_idx), cols, kmax)
    out = np.empty(len(row_ptr) - 1)
    for i in range(len(row_ptr) - 1):
        if bad[i] or e[i] == NONFINITE or f == NONFINITE:
            out[i] = math.nan
            continue
        acc = 0
        for p in range(row_ptr[i], row_ptr[i + 1]):
            acc += (ozaki2.scaled_integer(float(vals[p]), int(e[i])) *
                    ozaki2.scaled_integer(float(x[col_idx[p]]), f))
        out[i] = ozaki2.round_scaled(acc, int(e[i]) + f)
    return out
