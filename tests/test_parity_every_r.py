"""GPU parity for every number of moduli r = 1..20 against the CPU oracle.

Several kernels are compiled once per r, or per pass of moduli, with that r's constants
(the CRT's digit table and limb count, the SpMV row pass, the on-the-fly GEMV residue
passes), so each r is its own code.  This file runs every such instantiation at least
once, element by element against the oracle (<= 2 ulp, expected bit-exact):

* the CRT reconstruction on extreme values (X = +-2^Q, rounding ties, subnormal and
  overflowing results, NaN exponents) for r = 1..20, and on values next to the points
  where its rounding of both signs changes level, for r with 2, 3 and 4 limbs;
* the whole emulated DGEMM for r = 1..20 on wide-range operands;
* the widest scaled integers the budget allows (r = 20 with k = 1 and 2: 76-bit widths)
  through ozk_deconstruct, ozk_dgemm (both scaling rules) and ozk_dgemv;
* the on-the-fly GEMV in each residue-pass kernel the dispatch can reach (narrow and
  wide residue arithmetic, one or two 16-column tiles, first pass of up to 16 moduli and
  the second pass for r = 17..20) and the base-256 digits kernel for every count of
  32-column tiles (1..8) and every r that takes it;
* the emulated SpMV for r = 1..20 on the 7-point operator, and a diagonal matrix (one
  entry per row, the widest budget) for r = 14..20.
"""
import numpy as np
import pytest
import torch

import fp64_gemm_emulation_ozk_amd as ozk
import ozk_inputs
from oracle import ozaki2, rns, spmv

from gpu_common import announce, assert_within_ulps, to_dev

pytestmark = pytest.mark.gpu

ALL_R = list(range(1, 21))


def _k_for(r: int, want: int) -> int:
    """The largest k <= want that leaves r moduli a bit budget of at least 4 bits."""
    k = want
    while rns.budget_q(r) - rns.ceil_log2(k) < 4:
        k //= 2
    return max(k, 1)


@pytest.mark.parametrize("r", ALL_R)
def test_reconstruct_extremes_every_r(r):
    """X = 0, +-1, +-2^Q (the ends of the range the budget keeps every dot product in),
    random values, 53-bit rounding ties with and without lower digits, folded into
    [-2^Q, 2^Q]; shifts that give subnormal, overflowing and ordinary results; one NaN
    exponent.  Products arrive as arbitrary int32 representatives of their residues."""
    announce(f"reconstruct extremes r={r}")
    ms = rns.moduli(r)
    half = 2 ** rns.budget_q(r)
    rng = np.random.default_rng(100 + r)
    xs = [0, 1, -1, half, -half, half - 1, -(half - 1), 3, -5]
    xs += [int(v) for v in rng.integers(-2**62, 2**62, size=24)]
    xs += [int.from_bytes(rng.bytes(20), "little") - 2**159 for _ in range(24)]
    ties = [2**93 + 2**40, 2**93 + 2**40 + 1, -(2**93 + 2**40 + 1), 2**53 + 1, 2**53 + 3,
            (2**53 + 1) * 2**40 + 7, 2**80 + 2**27, 2**80 + 2**27 + 5, 2**101 + 2**48 + 3,
            2**140 + 2**87, -(2**150 + 2**97 + 1)]
    xs += ties
    xs = [((x + half) % (2 * half + 1)) - half for x in xs]
    n = len(xs)
    shifts = [int(v) for v in rng.integers(-900, 1200, size=n)]
    shifts[:6] = [0, 1075, 1074, -970, 60, 1100]
    prods = np.empty((r, 1, n), dtype=np.int64)
    for j, x in enumerate(xs):
        for l, m in enumerate(ms):
            prods[l, 0, j] = (x % m) + m * int(rng.integers(-8000, 8000))
    e = np.array([0], dtype=np.int64)
    f = np.array(shifts, dtype=np.int64)
    f[-1] = ozaki2.NONFINITE
    got = ozk.ozk_reconstruct(to_dev(prods.astype(np.int32)), to_dev(e.astype(np.int32)),
                              to_dev(f.astype(np.int32)))
    torch.cuda.synchronize()
    want = ozaki2.reconstruct(prods, r, e, f)
    assert assert_within_ulps(got.cpu().numpy(), want, 0) == 0


def _fold_boundary_values(rng, q):
    """Integers |X| <= 2^q that stress the CRT's rounding of both signs: X around v 2^80
    and v 2^120 for v next to +-8192 (where the folded top digits leave 13 bits), with
    lower digits that are zero, half a unit or random; midpoints above and below negative
    powers of two with and without a nonzero tail; negative ties of odd and even
    mantissas."""
    xs = []
    for shift in (40, 80, 120):
        for v in (-8194, -8193, -8192, -8191, -8190, 8190, 8191, 8192, 8193):
            for low in (0, 1, 1 << (shift - 1), (1 << shift) - 1,
                        int.from_bytes(rng.bytes(16), "little") % (1 << shift)):
                xs.append(v * (1 << shift) + low)
    for k in (54, 60, 93, 100, 121, 133):
        p2 = 1 << k
        mid_up = -p2 + (1 << (k - 54))        # halfway to the next double towards zero
        xs += [mid_up, mid_up + 1, mid_up - 1, -p2, -p2 + 1, -p2 - 1]
        mid_dn = -p2 - (1 << (k - 53))        # halfway to the next double away from zero
        xs += [mid_dn, mid_dn + 1, mid_dn - 1]
        odd = -(p2 + (1 << (k - 52)) + (1 << (k - 53)))   # tie next to an odd mantissa
        xs += [odd, odd + 1, odd - 1]
    return [x for x in xs if abs(x) <= 1 << q]


@pytest.mark.parametrize("r", [9, 10, 11, 12, 13, 15, 16, 17, 18, 20])
def test_reconstruct_signed_rounding(r):
    """The CRT rounds both signs from carried digits, folding the top digits until the
    value has 54 bits; X on and next to the fold boundaries, negative ties and midpoints
    next to negative powers of two must round exactly as the oracle's exact rounding, for
    r with 2, 3 and 4 limbs, with and without a top digit beyond 13 bits.  Shifts keep
    the results normal (other tests cover subnormal and overflowing ones)."""
    announce(f"reconstruct signed rounding r={r}")
    ms = rns.moduli(r)
    rng = np.random.default_rng(700 + r)
    xs = _fold_boundary_values(rng, rns.budget_q(r))
    n = len(xs)
    assert n > 20
    prods = np.empty((r, 1, n), dtype=np.int64)
    for j, x in enumerate(xs):
        for l, m in enumerate(ms):
            prods[l, 0, j] = (x % m) + m * int(rng.integers(-8000, 8000))
    e = np.array([0], dtype=np.int64)
    f = rng.integers(-200, 200, size=n).astype(np.int64)
    got = ozk.ozk_reconstruct(to_dev(prods.astype(np.int32)), to_dev(e.astype(np.int32)),
                              to_dev(f.astype(np.int32)))
    torch.cuda.synchronize()
    want = ozaki2.reconstruct(prods, r, e, f)
    assert assert_within_ulps(got.cpu().numpy(), want, 0) == 0


@pytest.mark.parametrize("r", ALL_R)
def test_dgemm_every_r(r):
    """70 x 45 outputs, k up to 300 (less where r moduli leave no budget for it), entries
    (U - 0.5) exp(4 N): the whole path (deconstruction, residue products, CRT) for r."""
    k = _k_for(r, 300)
    announce(f"dgemm every r: r={r} k={k}")
    a, b = ozk_inputs.gemm_operands(70, 45, k, seed=500 + r, dist="phi", phi=4.0)
    got = ozk.ozk_dgemm(to_dev(a), to_dev(b), r)
    torch.cuda.synchronize()
    want = ozaki2.dgemm(a, b, r)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


@pytest.mark.parametrize("k", [1, 2])
def test_widest_budget_deconstruct(k):
    """r = 20 with k = 1 or 2: both widths are 76 bits, so scaled integers reach 2^76, the
    end of the residue arithmetic's exact range; planes and exponents bit-exact."""
    r = 20
    assert rns.scaling_bits(r, k) == (76, 76)
    rng = np.random.default_rng(60 + k)
    for axis in (0, 1):
        announce(f"deconstruct widest budget r={r} k={k} axis={axis}")
        shape = (300, k) if axis == 0 else (k, 300)
        x = ozk_inputs.phi_matrix(rng, shape, 4.0)
        if axis == 0:
            x[0, 0] = np.nextafter(1.0, 2.0)     # scales to just above 2^75
            x[1, 0] = -np.nextafter(2.0, 0.0)    # rounds up to -2^76
        else:
            x[0, 0] = np.nextafter(1.0, 2.0)
            x[0, 1] = -np.nextafter(2.0, 0.0)
        planes, exps = ozk.ozk_deconstruct(to_dev(x), axis, r)
        torch.cuda.synchronize()
        want_e = ozaki2.scale_exponents(x, 76, axis)
        np.testing.assert_array_equal(exps.cpu().numpy().astype(np.int64), want_e)
        want_pl = ozaki2.residue_planes(x, want_e, r, axis)
        np.testing.assert_array_equal(planes.cpu().numpy()[:, :, :k], want_pl)


@pytest.mark.parametrize("rule", ["max", "norm"])
@pytest.mark.parametrize("k", [1, 2])
def test_widest_budget_dgemm(k, rule):
    r = 20
    announce(f"dgemm widest budget r={r} k={k} {rule}")
    a, b = ozk_inputs.gemm_operands(130, 70, k, seed=70 + k, dist="phi", phi=4.0)
    a[0, 0], b[0, 0] = np.nextafter(2.0, 0.0), -np.nextafter(2.0, 0.0)
    got = ozk.ozk_dgemm_ex(to_dev(a), to_dev(b), r, rule)
    torch.cuda.synchronize()
    want = ozaki2.dgemm(a, b, r, scaling=rule)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0
    if rule == "max":
        np.testing.assert_array_equal(got.cpu().numpy(), ozaki2.exact_scaled_product(a, b, r))


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("k,nrhs", [(1, 1), (2, 3), (1, 32), (2, 20)])
def test_widest_budget_dgemv(k, nrhs, mode):
    r = 20
    announce(f"dgemv widest budget r={r} k={k} nrhs={nrhs} mode={mode}")
    a, x = ozk_inputs.gemv_operands(140, k, nrhs, seed=80 + k + nrhs)
    a[3, 0] = np.nextafter(2.0, 0.0)
    da, dx = to_dev(a), to_dev(x)
    if mode == 0:
        got = ozk.ozk_dgemv(da, dx, r, mode=0)
    else:
        planes, exps = ozk.ozk_deconstruct(da, 0, r, k_budget=k)
        got = ozk.ozk_dgemv(None, dx, r, mode=1, a_planes=planes, a_exps=exps)
    torch.cuda.synchronize()
    want = ozaki2.dgemv(a, x, r)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


def gemv_fly_kernels(r: int, k: int, nrhs: int):
    """The on-the-fly kernels a GEMV call launches, as (wide, first modulus, moduli in
    the pass, 16-column tiles), or [] when it takes the base-256 digits kernel: digits
    when P_A <= 50 and r * nrhs <= 256; residues with the wide arithmetic when P_A > 51;
    passes of at most 16 moduli."""
    pa, _ = rns.scaling_bits(r, k)
    if pa <= 50 and r * nrhs <= 256:
        return []
    wide, ct = pa > 51, (1 if nrhs <= 16 else 2)
    out = [(wide, 0, min(r, 16), ct)]
    if r > 16:
        out.append((wide, 16, r - 16, ct))
    return out


# One case per on-the-fly kernel the dispatch can reach (23 of them): (r, k, nrhs).
FLY_CASES = [
    (9, 700, 32), (10, 700, 26), (11, 700, 24), (12, 700, 22), (13, 700, 20),
    (14, 100, 1), (14, 100, 17),                  # narrow (P_A = 51), r = 14, 1 and 2 tiles
    (15, 8193, 1), (15, 8193, 18),                # narrow (P_A = 51), r = 15
    (14, 20, 3), (14, 32, 32),                    # wide, r = 14
    (15, 300, 16), (15, 300, 31),                 # wide, r = 15
    (16, 1000, 2), (16, 1000, 17),                # wide, r = 16
    (17, 600, 5), (17, 600, 32),                  # wide, second pass of 1 modulus
    (18, 4100, 16), (18, 4100, 19),               # 2 moduli
    (19, 257, 1), (19, 257, 25),                  # 3 moduli
    (20, 900, 7), (20, 900, 32),                  # 4 moduli
]


def test_fly_cases_cover_every_reachable_kernel():
    reached = set()
    for r, k, nrhs in FLY_CASES:
        kernels = gemv_fly_kernels(r, k, nrhs)
        assert kernels, (r, k, nrhs)
        reached.update(kernels)
    every = set()
    for r in ALL_R:
        for nrhs in range(1, 33):
            for lk in range(18):
                k = min(1 << lk, 131071)
                try:
                    every.update(gemv_fly_kernels(r, k, nrhs))
                except ValueError:
                    pass
    assert reached == every and len(every) == 23


@pytest.mark.parametrize("r,k,nrhs", FLY_CASES)
def test_dgemv_fly_kernel_matches_oracle(r, k, nrhs):
    announce(f"dgemv fly r={r} k={k} nrhs={nrhs} kernels={gemv_fly_kernels(r, k, nrhs)}")
    a, x = ozk_inputs.gemv_operands(140, k, nrhs, seed=r * 1000 + nrhs)
    a[5] *= 2.0 ** -40
    got = ozk.ozk_dgemv(to_dev(a), to_dev(x), r, mode=0)
    torch.cuda.synchronize()
    want = ozaki2.dgemv(a, x, r)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


def _fast_k(r, k, nrhs):
    """A multiple of 32 near k that reaches the same on-the-fly kernels (the kernels take an
    unconditional-load path when k is a multiple of 32 and the rows are 16-byte aligned)."""
    want = gemv_fly_kernels(r, k, nrhs)
    for kk in (k // 32 * 32, (k + 31) // 32 * 32, (k // 32 + 2) * 32, (k // 32 - 1) * 32):
        if kk > 0 and gemv_fly_kernels(r, kk, nrhs) == want:
            return kk
    raise AssertionError((r, k, nrhs))


# The same 23 kernels on their unconditional-load path (k a multiple of 32).
FLY_FAST_CASES = [(r, _fast_k(r, k, nrhs), nrhs) for r, k, nrhs in FLY_CASES]


def test_fly_fast_cases_cover_every_reachable_kernel():
    reached = set()
    for r, k, nrhs in FLY_FAST_CASES:
        assert k % 32 == 0
        reached.update(gemv_fly_kernels(r, k, nrhs))
    assert len(reached) == 23


@pytest.mark.parametrize("r,k,nrhs", FLY_FAST_CASES)
def test_dgemv_fly_fast_path_matches_oracle(r, k, nrhs):
    """Rows of 16-byte aligned fp64 and k % 32 == 0; a row holding a NaN, a row scaled far
    down, and K padded past k when k is an odd multiple of 32."""
    announce(f"dgemv fly fast r={r} k={k} nrhs={nrhs} kernels={gemv_fly_kernels(r, k, nrhs)}")
    a, x = ozk_inputs.gemv_operands(140, k, nrhs, seed=r * 1000 + nrhs + 7)
    a[5] *= 2.0 ** -40
    a[9, k // 2] = np.nan
    got = ozk.ozk_dgemv(to_dev(a), to_dev(x), r, mode=0)
    torch.cuda.synchronize()
    want = ozaki2.dgemv(a, x, r)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


# Base-256 digits path for every r that takes it (1..15), every count of 16-column tiles
# (1..16, each instantiated with its own tile count), full and partial last tiles.
DIGIT_CASES = [(1, 10, 16), (2, 700, 16), (3, 700, 16), (4, 700, 16), (5, 700, 16),
               (6, 700, 16), (7, 700, 16), (8, 700, 16), (9, 700, 16), (10, 700, 16),
               (11, 700, 16), (12, 700, 16), (13, 700, 16), (14, 700, 16), (15, 16385, 16),
               (8, 700, 32), (3, 700, 5), (9, 700, 3), (13, 700, 12), (14, 700, 8)]


@pytest.mark.parametrize("r,k,nrhs", DIGIT_CASES)
def test_dgemv_digits_every_r(r, k, nrhs):
    assert gemv_fly_kernels(r, k, nrhs) == []
    announce(f"dgemv digits r={r} k={k} nrhs={nrhs} tiles={(r * nrhs + 15) // 16}")
    a, x = ozk_inputs.gemv_operands(150, k, nrhs, seed=r * 77 + nrhs)
    got = ozk.ozk_dgemv(to_dev(a), to_dev(x), r, mode=0)
    planes, exps = ozk.ozk_deconstruct(to_dev(a), 0, r, k_budget=k)
    got_st = ozk.ozk_dgemv(None, to_dev(x), r, mode=1, a_planes=planes, a_exps=exps)
    torch.cuda.synchronize()
    want = ozaki2.dgemv(a, x, r)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0
    assert assert_within_ulps(got_st.cpu().numpy(), want, 2) == 0


def test_digit_cases_cover_every_tile_count():
    tiles = {(r * nrhs + 15) // 16 for r, _, nrhs in DIGIT_CASES}
    assert tiles == set(range(1, 17))
    assert any(r * nrhs % 16 for r, _, nrhs in DIGIT_CASES)
    assert {r for r, _, _ in DIGIT_CASES} == set(range(1, 16))


@pytest.mark.parametrize("r", ALL_R)
def test_spmv_poisson_every_r(r):
    """The 7-point operator on a 6^3 grid (216 rows of up to 7 entries), x with a wide
    range, for each r (its row pass is compiled per r)."""
    n = 6
    announce(f"spmv poisson every r: r={r}")
    rp, ci, v = ozk_inputs.poisson_7pt_csr(n)
    x = ozk_inputs.phi_matrix(np.random.default_rng(900 + r), (n ** 3, 1), 3.0)[:, 0]
    got = ozk.ozk_spmv_csr(to_dev(rp), to_dev(ci), to_dev(v), to_dev(x), r, 7)
    torch.cuda.synchronize()
    want = spmv.spmv_csr(rp, ci, v, x, r, 7)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


@pytest.mark.parametrize("r", [14, 15, 16, 17, 18, 19, 20])
def test_spmv_diagonal_widest_budget(r):
    """A diagonal matrix (one entry per row, kmax = 1): the largest widths of each r (76
    bits at r = 20), through the wide residue arithmetic of the row pass."""
    rows = 700
    announce(f"spmv diagonal r={r}")
    rng = np.random.default_rng(950 + r)
    rp = np.arange(rows + 1, dtype=np.int32)
    ci = rng.permutation(rows).astype(np.int32)
    v = ozk_inputs.phi_matrix(rng, (1, rows), 4.0)[0]
    v[0] = np.nextafter(2.0, 0.0)
    x = ozk_inputs.phi_matrix(rng, (rows, 1), 4.0)[:, 0]
    got = ozk.ozk_spmv_csr(to_dev(rp), to_dev(ci), to_dev(v), to_dev(x), r, 1)
    torch.cuda.synchronize()
    want = spmv.spmv_csr(rp, ci, v, x, r, 1)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0
