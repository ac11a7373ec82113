"""Seeded synthetic input generators shared by the tests, the oracle checks and the bench.

This module holds only random-number draws; none of the emulation arithmetic lives
here.  Every generator takes an explicit seed and draws with
``numpy.random.default_rng(seed)`` (PCG64) in a fixed order (A, then B or X), so the
oracle and the GPU path always see bit-identical operands.

Distributions (all from the workload descriptions of the emulated-fp64 GEMM/GEMV and
the exact INT8 product):

* ``uniform``:   entries U(-1, 1).
* ``phi``:       entries (U(0,1) - 0.5) * exp(phi * N(0,1)); phi = 0.5 (moderate range)
                 or phi = 4 (wide dynamic range).
* ``int8``:      integers uniform in [-128, 127].
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "uniform_matrix",
    "phi_matrix",
    "int8_matrix",
    "gemm_operands",
    "gemv_operands",
    "int8_operands",
    "small_int_matrix",
]


def uniform_matrix(rng: np.random.Generator, shape) -> np.ndarray:
    """Entries drawn from U(-1, 1), float64, C-contiguous."""
    return rng.uniform(-1.0, 1.0, size=shape)


def phi_matrix(rng: np.random.Generator, shape, phi: float) -> np.ndarray:
    """Entries (U(0,1) - 0.5) * exp(phi * N(0,1)): U is drawn first, then N."""
    u = rng.random(shape)
    g = rng.standard_normal(shape)
    return (u - 0.5) * np.exp(phi * g)


def int8_matrix(rng: np.random.Generator, shape) -> np.ndarray:
    """Integers uniform in [-128, 127], int8."""
    return rng.integers(-128, 128, size=shape, dtype=np.int8)


def small_int_matrix(rng: np.random.Generator, shape, bound: int) -> np.ndarray:
    """Integer-valued float64 entries uniform in [-bound, bound]."""
    return rng.integers(-bound, bound + 1, size=shape).astype(np.float64)


def gemm_operands(m: int, n: int, k: int, seed: int, dist: str = "uniform", phi: float = 0.5):
    """A (m x k) and B (k x n), float64 row-major, drawn A first then B."""
    rng = np.random.default_rng(seed)
    if dist == "uniform":
        a = uniform_matrix(rng, (m, k))
        b = uniform_matrix(rng, (k, n))
    elif dist == "phi":
        a = phi_matrix(rng, (m, k), phi)
        b = phi_matrix(rng, (k, n), phi)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return a, b


def gemv_operands(m: int, k: int, nrhs: int, seed: int):
    """A (m x k) and X (k x nrhs), both U(-1, 1), drawn A first then X."""
    rng = np.random.default_rng(seed)
    a = uniform_matrix(rng, (m, k))
    x = uniform_matrix(rng, (k, nrhs))
    return a, x


def int8_operands(m: int, n: int, k: int, seed: int):
    """A (m x k) and B (k x n), int8 uniform in [-128, 127], drawn A first then B."""
    rng = np.random.default_rng(seed)
    a = int8_matrix(rng, (m, k))
    b = int8_matrix(rng, (k, n))
    return a, b


def int4_int8_operands(m: int, n: int, k: int, seed: int):
    """A (m x k) int4 uniform in [-8, 7], one value per int8 byte, and B (k x n) int8
    uniform in [-128, 127], drawn A first then B."""
    rng = np.random.default_rng(seed)
    a = rng.integers(-8, 8, size=(m, k), dtype=np.int8)
    b = int8_matrix(rng, (k, n))
    return a, b


def uniform_matrix_device(shape, seed: int, device):
    """Entries U(-1, 1) as float64 drawn on a GPU by torch's seeded generator (for
    operands too large to draw on the host); the same seed gives the same matrix."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.rand(shape, generator=gen, dtype=torch.float64, device=device) * 2.0 - 1.0


def poisson_7pt_csr(n: int):
    """The 7-point operator 6 u_p - (sum of the grid neighbours of p) on an n x n x n
    grid with neighbours outside the grid dropped, rows in lexicographic order (i, j, k)
    and columns ascending within each row: (row_ptr int32, col_idx int32, vals float64)."""
    N = n ** 3
    p = np.arange(N, dtype=np.int64)
    i, j, k = p // (n * n), (p // n) % n, p % n
    # offsets in ascending column order
    offs = [(-n * n, i > 0), (-n, j > 0), (-1, k > 0), (0, np.ones(N, dtype=bool)),
            (1, k < n - 1), (n, j < n - 1), (n * n, i < n - 1)]
    cols = np.stack([p + d for d, _ in offs], axis=1)
    valid = np.stack([m for _, m in offs], axis=1)
    vals = np.where(np.arange(7)[None, :] == 3, 6.0, -1.0) * np.ones((N, 1))
    row_ptr = np.concatenate([[0], np.cumsum(valid.sum(axis=1))]).astype(np.int32)
    return row_ptr, cols[valid].astype(np.int32), vals[valid].astype(np.float64)


def random_csr(rows: int, cols: int, max_len: int, seed: int, phi: float = 0.0):
    """A CSR matrix with row lengths uniform in [0, max_len] (some rows empty), distinct
    ascending column indices per row, values U(-1,1) (phi = 0) or (U - 0.5) exp(phi N)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, max_len + 1, size=rows)
    row_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    col_idx = np.concatenate([np.sort(rng.choice(cols, size=L, replace=False)) for L in lens]
                             ) if rows else np.zeros(0)
    nnz = int(row_ptr[-1])
    vals = (phi_matrix(rng, (1, nnz), phi)[0] if phi > 0 else uniform_matrix(rng, (1, nnz))[0])
    return row_ptr, col_idx.astype(np.int32), vals
