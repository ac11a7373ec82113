"""GPU parity of the emulated SpMV (CSR) against the CPU oracle, element by element:
the 7-point Poisson operator and random CSR matrices over narrow and wide scaling, the
rows the reading defines (empty, Inf, too long, a bad column index, a bad row extent,
NaN in x), the operator's closed form, and a 128^3 grid on sampled rows."""
import numpy as np
import pytest
import torch

import fp64_gemm_emulation_ozk_amd as ozk
import ozk_inputs
from oracle import spmv

from gpu_common import announce, assert_within_ulps, to_dev

pytestmark = pytest.mark.gpu


def _run(rp, ci, v, x, r, kmax):
    y = ozk.ozk_spmv_csr(to_dev(rp.astype(np.int32)), to_dev(ci.astype(np.int32)),
                         to_dev(v.astype(np.float64)), to_dev(x), r, kmax)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("n,r", [(16, 8), (16, 14), (16, 16), (12, 20), (3, 5)])
def test_spmv_poisson_matches_oracle(n, r):
    announce(f"spmv poisson n={n} r={r}")
    rp, ci, v = ozk_inputs.poisson_7pt_csr(n)
    x = ozk_inputs.uniform_matrix(np.random.default_rng(n + r), (n ** 3, 1))[:, 0]
    got = _run(rp, ci, v, x, r, 7)
    want = spmv.spmv_csr(rp, ci, v, x, r, 7)
    assert assert_within_ulps(got, want, 2) == 0


@pytest.mark.parametrize("rows,cols,kmax,r,phi", [(3000, 2000, 40, 14, 4.0),
                                                   (1000, 5000, 100, 20, 2.0),
                                                   (777, 333, 9, 12, 0.0),
                                                   (64, 1, 1, 6, 1.0)])
def test_spmv_random_csr_matches_oracle(rows, cols, kmax, r, phi):
    announce(f"spmv random rows={rows} cols={cols} kmax={kmax} r={r}")
    rp, ci, v = ozk_inputs.random_csr(rows, cols, kmax, seed=rows + r, phi=phi)
    x = ozk_inputs.phi_matrix(np.random.default_rng(cols), (cols, 1), 2.0)[:, 0]
    got = _run(rp, ci, v, x, r, kmax)
    want = spmv.spmv_csr(rp, ci, v, x, r, kmax)
    assert assert_within_ulps(got, want, 2) == 0


def test_spmv_special_rows():
    """Empty row (+0), Inf in a row, a row longer than kmax, an out-of-range column and a
    row extent past nnz (all NaN, nothing read through them), then NaN in x."""
    announce("spmv special rows")
    rp = np.array([0, 0, 2, 4, 7, 9, 10, 40], dtype=np.int32)
    ci = np.array([0, 3, 1, 2, 0, 1, 2, 1, 1 << 30, 2], dtype=np.int32)
    v = np.array([1.0, 2.0, np.inf, 1.0, 1.0, 1.0, 1.0, 3.0, 4.0, 0.5])
    x = np.array([1.0, -2.0, 0.5, 0.25])
    got = _run(rp, ci, v, x, 8, 2)
    assert got[0] == 0.0 and not np.signbit(got[0])
    assert got[1] == 1.5
    assert np.all(np.isnan(got[[2, 3, 4, 6]]))
    assert got[5] == 0.25
    # the oracle agrees wherever the extents are valid
    want = spmv.spmv_csr(rp[:7], ci[:10], v[:10], x, 8, 2)
    assert assert_within_ulps(got[:6], want[:6], 0) == 0
    xs = x.copy()
    xs[1] = np.nan
    assert np.all(np.isnan(_run(rp[:6], ci[:9], v[:9], xs, 8, 3)))


def test_spmv_poisson_quadratic_closed_form():
    announce("spmv poisson closed form")
    n = 20
    rp, ci, v = ozk_inputs.poisson_7pt_csr(n)
    g = np.arange(n, dtype=np.float64)
    u = (g[:, None, None] ** 2 + g[None, :, None] ** 2 + g[None, None, :] ** 2).reshape(-1)
    y = _run(rp, ci, v, u, 10, 7).reshape(n, n, n)
    np.testing.assert_array_equal(y[1:-1, 1:-1, 1:-1], -6.0)


def test_spmv_poisson_128_sampled():
    """The 128^3 grid (2.1 M rows, 14.6 M entries) at r = 16, sampled rows against the
    oracle (x's exponent from all of x)."""
    announce("spmv poisson 128^3 sampled")
    n = 128
    rp, ci, v = ozk_inputs.poisson_7pt_csr(n)
    x = ozk_inputs.phi_matrix(np.random.default_rng(5), (n ** 3, 1), 1.0)[:, 0]
    got = _run(rp, ci, v, x, 16, 7)
    rng = np.random.default_rng(6)
    rows = np.sort(np.concatenate([rng.choice(n ** 3, 300, replace=False), [0, n ** 3 - 1]]))
    want = spmv.spmv_csr(rp, ci, v, x, 16, 7, rows=rows)
    assert assert_within_ulps(got[rows], want, 2) == 0


def test_spmv_blocks_staged_and_direct():
    """Row blocks of 256 whose entries fit the workgroup's LDS staging (short rows) next to
    blocks that do not (long rows), in one matrix, against the oracle."""
    announce("spmv staged and direct blocks")
    r, kmax, cols = 14, 40, 3000
    rp1, ci1, v1 = ozk_inputs.random_csr(600, cols, 6, seed=31, phi=1.0)
    rp2, ci2, v2 = ozk_inputs.random_csr(500, cols, kmax, seed=32, phi=1.0)
    rp = np.concatenate([rp1, rp2[1:] + rp1[-1]]).astype(np.int32)
    ci = np.concatenate([ci1, ci2]).astype(np.int32)
    v = np.concatenate([v1, v2])
    x = ozk_inputs.phi_matrix(np.random.default_rng(33), (cols, 1), 2.0)[:, 0]
    got = _run(rp, ci, v, x, r, kmax)
    want = spmv.spmv_csr(rp, ci, v, x, r, kmax)
    assert assert_within_ulps(got, want, 2) == 0


def test_spmv_non_monotone_row_ptr():
    """Rows whose extents leave the range their workgroup staged (row_ptr not monotone)
    read their entries from global memory; a row with end < start is malformed (NaN).
    Each well-formed row must equal the oracle on the same entries laid out in order."""
    announce("spmv non-monotone row_ptr")
    r, kmax = 12, 16
    rng = np.random.default_rng(41)
    nnz, cols = 40, 30
    ci = rng.integers(0, cols, size=nnz).astype(np.int32)
    v = ozk_inputs.uniform_matrix(rng, (1, nnz))[0]
    # the workgroup stages entries [2, 20): rows 0 and 3 lie inside, row 2 starts before
    # it (read from global memory), row 1 is reversed
    rp = np.array([2, 9, 1, 6, 20], dtype=np.int32)
    x = ozk_inputs.uniform_matrix(rng, (cols, 1))[:, 0]
    got = _run(rp, ci, v, x, r, kmax)
    assert np.isnan(got[1])
    for i in (0, 2, 3):
        s, t = int(rp[i]), int(rp[i + 1])
        want = spmv.spmv_csr(np.array([0, t - s]), ci[s:t], v[s:t], x, r, kmax)
        assert assert_within_ulps(got[i:i + 1], want, 2) == 0
