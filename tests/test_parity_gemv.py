"""GPU parity of the emulated GEMV / low-batch GEMV (both modes) against the CPU oracle.

On the fly (A streamed as fp64, residues formed in registers) and stored (A's residue
planes from ozk_deconstruct) must both equal the oracle's emulated product element by
element (<= 2 ulp, expected bit-exact), for 1..32 right-hand sides, ragged sizes, r up to
20 (more than 16 moduli takes two on-the-fly passes), special rows, and the full
32768 x 32768 configuration on sampled rows."""
import numpy as np
import pytest
import torch

import fp64_gemm_emulation_ozk_amd as ozk
import ozk_inputs
from oracle import ozaki2, reference

from gpu_common import announce, assert_within_ulps, to_dev

pytestmark = pytest.mark.gpu


def _run(a, x, r, mode, cached_exps=False):
    da, dx = to_dev(a), to_dev(x)
    if mode == 1:
        planes, exps = ozk.ozk_deconstruct(da, 0, r, k_budget=a.shape[1])
        return ozk.ozk_dgemv(None, dx, r, mode=1, a_planes=planes, a_exps=exps)
    exps = None
    if cached_exps:
        _, exps = ozk.ozk_deconstruct(da, 0, r, k_budget=a.shape[1])
    return ozk.ozk_dgemv(da, dx, r, mode=0, a_exps=exps)


CASES = [
    # m, k, nrhs, r
    (300, 257, 1, 14),
    (300, 257, 8, 16),
    (129, 1000, 32, 14),
    (65, 64, 3, 8),
    (1, 1, 1, 5),
    (200, 300, 5, 20),
    (257, 4100, 32, 18),
    # on-the-fly residue path (r * nrhs > 256) with a partly filled second 16-column tile
    (130, 700, 20, 14),
    (97, 333, 17, 16),
]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("m,k,nrhs,r", CASES)
def test_dgemv_matches_oracle(m, k, nrhs, r, mode):
    announce(f"dgemv m={m} k={k} nrhs={nrhs} r={r} mode={mode}")
    a, x = ozk_inputs.gemv_operands(m, k, nrhs, seed=m + k + nrhs)
    got = _run(a, x, r, mode)
    torch.cuda.synchronize()
    want = ozaki2.dgemv(a, x, r)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


def test_dgemv_cached_exponents_equal_computed():
    announce("dgemv cached exps")
    a, x = ozk_inputs.gemv_operands(190, 513, 4, seed=3)
    g1 = _run(a, x, 14, 0, cached_exps=True)
    g2 = _run(a, x, 14, 0, cached_exps=False)
    torch.cuda.synchronize()
    assert torch.equal(g1.view(torch.int64), g2.view(torch.int64))


@pytest.mark.parametrize("mode", [0, 1])
def test_dgemv_special_rows(mode):
    announce(f"dgemv special rows mode={mode}")
    a, x = ozk_inputs.gemv_operands(100, 300, 4, seed=8)
    a = ozk_inputs.phi_matrix(np.random.default_rng(8), (100, 300), 4.0)
    a[3] = 0.0
    a[7, 11] = np.nan
    a[9] *= 1e-305
    x[5, 2] = np.inf
    got = _run(a, x, 16, mode)
    torch.cuda.synchronize()
    want = ozaki2.dgemv(a, x, 16)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


# The on-the-fly mode streams A through base-256 digits of the scaled integers when the
# row budget P_A is at most 50 bits and r * nrhs <= 256; these cases are chosen to take
# that path (P_A from the oracle's budget), with its edge cases: rows so small that the
# scale 2^e exceeds the fp64 range (e > 1023), zero and NaN rows, scaled integers of
# exactly +-2^P_A at P_A = 50, several K slices of 8192 with a ragged tail, and 8 column
# tiles.
def _digit_path(k, r, nrhs):
    from oracle import rns
    pa, _ = rns.scaling_bits(r, k)
    return pa <= 50 and r * nrhs <= 256


def test_dgemv_digits_special_rows():
    announce("dgemv digits special rows")
    m, k, nrhs, r = 100, 300, 4, 14
    assert _digit_path(k, r, nrhs)
    rng = np.random.default_rng(18)
    a = ozk_inputs.phi_matrix(rng, (m, k), 4.0)
    x = ozk_inputs.uniform_matrix(rng, (k, nrhs))
    a[3] = 0.0
    a[7, 11] = np.nan
    a[9] *= 1e-305          # e > 1023 for this row
    a[10] = 1e-320 * np.sign(a[10])   # subnormal row
    a[12, 5] = np.inf
    got = _run(a, x, r, 0)
    torch.cuda.synchronize()
    want = ozaki2.dgemv(a, x, r)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


def test_dgemv_digits_extreme_scaled_integers():
    announce("dgemv digits |a'| = 2^P_A")
    from oracle import rns
    m, k, nrhs, r = 40, 257, 2, 14
    pa, _ = rns.scaling_bits(r, k)
    assert pa == 50 and _digit_path(k, r, nrhs)
    rng = np.random.default_rng(19)
    a = ozk_inputs.uniform_matrix(rng, (m, k))
    x = ozk_inputs.uniform_matrix(rng, (k, nrhs))
    top = np.nextafter(2.0, 0.0)        # scales to 2^50 - 1/8, rounds to 2^50
    for i in range(m):
        a[i, (7 * i) % k] = (top if i % 2 == 0 else -top) * 2.0 ** (i - 20)
        a[i] = np.where(np.abs(a[i]) > abs(a[i, (7 * i) % k]), 0.0, a[i])
    got = _run(a, x, r, 0)
    torch.cuda.synchronize()
    want = ozaki2.dgemv(a, x, r)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


@pytest.mark.parametrize("m,k,nrhs,r", [(130, 2 * 8192 + 37, 2, 12), (70, 500, 18, 14),
                                        (33, 8192, 1, 10)])
def test_dgemv_digits_slices_and_tiles(m, k, nrhs, r):
    announce(f"dgemv digits m={m} k={k} nrhs={nrhs} r={r}")
    assert _digit_path(k, r, nrhs)
    a, x = ozk_inputs.gemv_operands(m, k, nrhs, seed=m + nrhs)
    got = _run(a, x, r, 0)
    torch.cuda.synchronize()
    want = ozaki2.dgemv(a, x, r)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


# The digits kernel's fast path (rows 16-byte aligned, k a multiple of 16): super-chunks
# past k inside the padding to 64, several K slices, ragged rows, special rows fed as they
# are (Inf/NaN rows must still give NaN), and several column-tile counts.
@pytest.mark.parametrize("m,k,nrhs,r", [(130, 720, 8, 14), (65, 2 * 8192 + 48, 2, 12),
                                        (200, 1024, 3, 14), (97, 656, 16, 14),
                                        (33, 16, 1, 9)])
def test_dgemv_digits_fast_path(m, k, nrhs, r):
    announce(f"dgemv digits fast path m={m} k={k} nrhs={nrhs} r={r}")
    assert _digit_path(k, r, nrhs) and k % 16 == 0
    a, x = ozk_inputs.gemv_operands(m, k, nrhs, seed=m + k + nrhs)
    got = _run(a, x, r, 0)
    torch.cuda.synchronize()
    want = ozaki2.dgemv(a, x, r)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


def test_dgemv_digits_fast_path_special_rows():
    announce("dgemv digits fast path special rows")
    m, k, nrhs, r = 100, 320, 4, 14
    assert _digit_path(k, r, nrhs)
    rng = np.random.default_rng(28)
    a = ozk_inputs.phi_matrix(rng, (m, k), 4.0)
    x = ozk_inputs.uniform_matrix(rng, (k, nrhs))
    a[3] = 0.0
    a[7, 11] = np.nan
    a[9] *= 1e-305          # e > 1023 for this row
    a[10] = 1e-320 * np.sign(a[10])   # subnormal row
    a[12, 5] = np.inf
    a[13, 319] = -np.inf    # in the last super-chunk
    got = _run(a, x, r, 0)
    torch.cuda.synchronize()
    want = ozaki2.dgemv(a, x, r)
    assert np.isnan(want[[7, 12, 13]]).all()
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


def test_dgemv_strided():
    announce("dgemv strided")
    a, x = ozk_inputs.gemv_operands(70, 90, 3, seed=2)
    abig = np.zeros((70, 96))
    abig[:, :90] = a
    xbig = np.zeros((90, 5))
    xbig[:, :3] = x
    da, dx = to_dev(abig)[:, :90], to_dev(xbig)[:, :3]
    out = torch.full((70, 4), 5.0, dtype=torch.float64, device=da.device)
    ozk.ozk_dgemv(da, dx, 14, mode=0, out=out[:, :3])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[:, 3] == 5.0)
    assert assert_within_ulps(got[:, :3], ozaki2.dgemv(a, x, 14), 2) == 0


@pytest.fixture(scope="module")
def big_gemv():
    """A 32768 x 32768, U(-1,1) (seed 4, drawn on the GPU) and X 32768 x 32 (seed 4,
    host); the 1- and 8-column cases use X's leading columns."""
    dev = torch.device("cuda:0")
    da = ozk_inputs.uniform_matrix_device((32768, 32768), 4, dev)
    x = ozk_inputs.uniform_matrix(np.random.default_rng(4), (32768, 32))
    return da, x


@pytest.mark.parametrize("nrhs", [1, 8, 32])
def test_dgemv_32768_sampled(big_gemv, nrhs):
    da, x = big_gemv
    r = 14
    announce(f"dgemv 32768^2 nrhs={nrhs} r={r} both modes, sampled rows")
    xs = np.ascontiguousarray(x[:, :nrhs])
    dx = to_dev(xs)
    y_fly = ozk.ozk_dgemv(da, dx, r, mode=0)
    planes, exps = ozk.ozk_deconstruct(da, 0, r, k_budget=32768)
    y_st = ozk.ozk_dgemv(None, dx, r, mode=1, a_planes=planes, a_exps=exps)
    torch.cuda.synchronize()
    del planes
    assert torch.equal(y_fly.view(torch.int64), y_st.view(torch.int64))
    rows = np.array([0, 1, 12345, 20000, 32767])
    a_rows = da[torch.as_tensor(rows, device=da.device)].cpu().numpy()
    want = ozaki2.dgemv(a_rows, xs, r)
    assert assert_within_ulps(y_fly.cpu().numpy()[rows], want, 2) == 0


def test_dgemv_32768_accuracy_r14_r16(big_gemv):
    """Normwise error against Dot2 on sampled rows: r = 14 is the configured size;
    r = 16 is the accuracy run (1e-15 needs 16 moduli at k = 32768 under the max rule)."""
    da, x = big_gemv
    rows = np.array([5, 777, 31000])
    a_rows = da[torch.as_tensor(rows, device=da.device)].cpu().numpy()
    xs = np.ascontiguousarray(x[:, :1])
    dd = reference.dot2_matmul(a_rows, xs)
    errs = {}
    for r in (14, 16):
        announce(f"dgemv 32768 accuracy r={r}")
        y = ozk.ozk_dgemv(da, to_dev(xs), r, mode=0).cpu().numpy()[rows]
        errs[r] = np.linalg.norm(y - dd) / np.linalg.norm(dd)
    assert errs[16] <= 1e-15
    assert errs[14] <= 1e-13
