"""GPU parity of the emulated DGEMM path against the CPU oracle, element by element.

Rows of the hot path covered: scale exponents and residue planes (bit-exact), int32
modular products (bit-exact), CRT reconstruction (bit-exact fp64; the stated bar is
<= 2 ulp), and the whole ozk_dgemm (<= 2 ulp of the oracle, expected bit-exact, and
normwise <= 1e-15 against the double-double reference at the tiny configuration)."""
import numpy as np
import pytest
import torch

import fp64_gemm_emulation_ozk_amd as ozk
import ozk_inputs
from oracle import ozaki2, reference, rns

from gpu_common import announce, assert_within_ulps, to_dev

pytestmark = pytest.mark.gpu


def _special_rows(x: np.ndarray, axis: int):
    """Plant a zero line, a subnormal line and a line with one huge entry."""
    x = x.copy()
    lines = x.shape[0] if axis == 0 else x.shape[1]
    if lines >= 4:
        sel = (lambda i: (i, slice(None))) if axis == 0 else (lambda i: (slice(None), i))
        x[sel(0)] = 0.0
        x[sel(1)] = x[sel(1)] * 1e-310
        x[sel(2)] = x[sel(2)] * 1e-300
        x[sel(3)][0] = 2.0**900
    return x


DECON_CASES = [
    # rows, cols, axis, r, dist
    (1, 1, 0, 14, "uniform"),
    (37, 100, 0, 14, "uniform"),
    (300, 257, 0, 16, "phi"),
    (130, 4100, 0, 20, "phi"),
    (5, 40000, 0, 14, "uniform"),     # long rows: two-pass path
    (100, 37, 1, 14, "uniform"),
    (257, 300, 1, 16, "phi"),
    (4100, 70, 1, 20, "phi"),
    (64, 64, 1, 8, "uniform"),
]


@pytest.mark.parametrize("rows,cols,axis,r,dist", DECON_CASES)
def test_deconstruct_bit_exact(rows, cols, axis, r, dist):
    announce(f"deconstruct rows={rows} cols={cols} axis={axis} r={r} {dist}")
    rng = np.random.default_rng(rows * 7 + cols)
    x = (ozk_inputs.phi_matrix(rng, (rows, cols), 4.0) if dist == "phi"
         else ozk_inputs.uniform_matrix(rng, (rows, cols)))
    x = _special_rows(x, axis)
    kdim = cols if axis == 0 else rows
    planes, exps = ozk.ozk_deconstruct(to_dev(x), axis, r)
    torch.cuda.synchronize()
    pa, pb = rns.scaling_bits(r, kdim)
    p = pa if axis == 0 else pb
    want_e = ozaki2.scale_exponents(x, p, axis)
    want_pl = ozaki2.residue_planes(x, want_e, r, axis)
    np.testing.assert_array_equal(exps.cpu().numpy().astype(np.int64), want_e)
    got = planes.cpu().numpy()
    np.testing.assert_array_equal(got[:, :, :kdim], want_pl)
    assert not np.any(got[:, :, kdim:]), "K padding must be zero"


def test_deconstruct_nonfinite_lines():
    announce("deconstruct nonfinite")
    x = ozk_inputs.uniform_matrix(np.random.default_rng(3), (6, 70))
    x[2, 5] = np.nan
    x[4, 0] = -np.inf
    planes, exps = ozk.ozk_deconstruct(to_dev(x), 0, 14)
    planes_t, exps_t = ozk.ozk_deconstruct(to_dev(x.T.copy()), 1, 14)
    torch.cuda.synchronize()
    e = exps.cpu().numpy()
    assert e[2] == ozaki2.NONFINITE and e[4] == ozaki2.NONFINITE
    np.testing.assert_array_equal(exps_t.cpu().numpy(), e)
    assert not np.any(planes.cpu().numpy()[:, [2, 4], :])
    np.testing.assert_array_equal(planes_t.cpu().numpy(), planes.cpu().numpy())


# The last two have more tiles (r * tiles_m * tiles_n) than the device has compute
# units, so workgroups walk several tiles: ragged and full tiles, 3 and 4 K pairs.
PRODUCT_CASES = [(1, 1, 64, 1), (300, 200, 256, 3), (257, 129, 64, 2), (512, 384, 640, 2),
                 (33, 700, 192, 4), (1030, 1030, 512, 11), (1024, 1280, 384, 13)]


@pytest.mark.parametrize("m,n,kp,r", PRODUCT_CASES)
def test_modular_products_bit_exact(m, n, kp, r):
    announce(f"modular_products m={m} n={n} kp={kp} r={r}")
    rng = np.random.default_rng(m + n + kp)
    pa = rng.integers(-128, 128, size=(r, m, kp), dtype=np.int8)
    pb = rng.integers(-128, 128, size=(r, n, kp), dtype=np.int8)
    pa[0, 0, :] = -128                 # extreme sums
    pb[0, 0, :] = -128
    got = ozk.ozk_modular_products(to_dev(pa), to_dev(pb))
    torch.cuda.synchronize()
    want = ozaki2.modular_products(pa, pb)
    np.testing.assert_array_equal(got.cpu().numpy().astype(np.int64), want)
    assert want[0, 0, 0] == kp * 2**14


RESIDUE_CASES = [(300, 200, 256, 20), (1, 1, 64, 1), (257, 130, 128, 16),
                 # several tiles per workgroup: ragged (3 pairs), full (2 and 8 pairs)
                 (1100, 900, 384, 16), (1536, 1280, 256, 12), (2048, 2048, 1024, 16)]


@pytest.mark.parametrize("m,n,kp,r", RESIDUE_CASES)
def test_modular_residues_bit_exact(m, n, kp, r):
    announce(f"modular_residues m={m} n={n} kp={kp} r={r}")
    rng = np.random.default_rng(m * n + kp)
    pa = rng.integers(-128, 128, size=(r, m, kp), dtype=np.int8)
    pb = rng.integers(-128, 128, size=(r, n, kp), dtype=np.int8)
    got = ozk.ozk_modular_residues(to_dev(pa), to_dev(pb))
    torch.cuda.synchronize()
    prods = ozaki2.modular_products(pa, pb)
    want = np.stack([(prods[l] + m_l // 2) % m_l - m_l // 2
                     for l, m_l in enumerate(rns.moduli(r))])
    np.testing.assert_array_equal(got.cpu().numpy().astype(np.int64), want)


@pytest.mark.parametrize("m,n,k,r,dist", [(40, 33, 100, 14, "uniform"), (64, 70, 300, 20, "phi"),
                                          (17, 5, 9, 8, "phi")])
def test_reconstruct_bit_exact(m, n, k, r, dist):
    announce(f"reconstruct m={m} n={n} k={k} r={r}")
    a, b = ozk_inputs.gemm_operands(m, n, k, seed=m * n, dist=dist, phi=4.0)
    pa_bits, pb_bits = rns.scaling_bits(r, k)
    e = ozaki2.scale_exponents(a, pa_bits, 0)
    f = ozaki2.scale_exponents(b, pb_bits, 1)
    prods = ozaki2.modular_products(ozaki2.residue_planes(a, e, r, 0),
                                    ozaki2.residue_planes(b, f, r, 1))
    got = ozk.ozk_reconstruct(to_dev(prods.astype(np.int32)), to_dev(e.astype(np.int32)),
                              to_dev(f.astype(np.int32)))
    torch.cuda.synchronize()
    want = ozaki2.reconstruct(prods, r, e, f)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


@pytest.mark.parametrize("r", [14, 16, 20, 5, 1])
def test_reconstruct_extremes(r):
    """Subnormal, overflowing and cancelling outputs, NaN exponents, raw int32 inputs
    (not reduced) and residues of X = +-2^Q, the end of the range the bit budget keeps
    every emulated dot product in."""
    announce(f"reconstruct extremes r={r}")
    ms = rns.moduli(r)
    half = 2 ** rns.budget_q(r)
    rng = np.random.default_rng(0)
    xs = [0, 1, -1, half, -half, half - 12345, 2**60 + 1, -(2**53 + 1), 2**53 + 3, 3, 5, 7]
    xs += [int(v) for v in rng.integers(-2**62, 2**62, size=20)]
    # exact midpoints of the 53-bit rounding, with and without nonzero lower digits
    ties = [2**93 + 2**40, 2**93 + 2**40 + 1, -(2**93 + 2**40 + 1), 2**53 + 1, 2**53 + 3,
            (2**53 + 1) * 2**40 + 7, 2**80 + 2**27, 2**80 + 2**27 + 5, 2**101 + 2**48 + 3]
    xs += ties
    # every X must lie in [-2^Q, 2^Q]: fold the ones a small r cannot hold
    xs = [((x + half) % (2 * half + 1)) - half for x in xs]
    shifts = [0, 1075, 1076, 1074, 1100, -970, -1000, 60, -10, 1075, 1075, 1075]
    shifts += [int(v) for v in rng.integers(-900, 1200, size=20)]
    shifts += [0, 0, 0, 0, 0, 40, 0, 3, 1100]
    n = len(xs)
    prods = np.empty((r, 1, n), dtype=np.int64)
    for j, x in enumerate(xs):
        for l, m in enumerate(ms):
            # any representative in int32 range: the kernel reduces it
            prods[l, 0, j] = (x % m) + m * int(rng.integers(-1000, 1000))
    e = np.array([0], dtype=np.int64)
    f = np.array(shifts, dtype=np.int64)
    f[-1] = ozaki2.NONFINITE
    got = ozk.ozk_reconstruct(to_dev(prods.astype(np.int32)), to_dev(e.astype(np.int32)),
                              to_dev(f.astype(np.int32)))
    torch.cuda.synchronize()
    want = ozaki2.reconstruct(prods, r, e, f)
    assert assert_within_ulps(got.cpu().numpy(), want, 0) == 0


DGEMM_CASES = [
    (64, 64, 64, 14, "uniform"),
    (1, 1, 1, 5, "uniform"),
    (300, 200, 257, 16, "phi"),
    (257, 129, 100, 12, "phi"),
    (513, 260, 70, 20, "phi"),
    (100, 300, 1000, 18, "uniform"),
]


@pytest.mark.parametrize("m,n,k,r,dist", DGEMM_CASES)
def test_dgemm_matches_oracle(m, n, k, r, dist):
    announce(f"dgemm m={m} n={n} k={k} r={r} {dist}")
    a, b = ozk_inputs.gemm_operands(m, n, k, seed=m + 2 * n + 3 * k, dist=dist, phi=4.0)
    got = ozk.ozk_dgemm(to_dev(a), to_dev(b), r)
    torch.cuda.synchronize()
    want = ozaki2.dgemm(a, b, r)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


def test_dgemm_special_lines():
    announce("dgemm special lines")
    a, b = ozk_inputs.gemm_operands(70, 65, 90, seed=9, dist="phi", phi=4.0)
    a = _special_rows(a, 0)
    b = _special_rows(b, 1)
    a[10, 3] = np.nan
    b[7, 20] = np.inf
    got = ozk.ozk_dgemm(to_dev(a), to_dev(b), 16)
    torch.cuda.synchronize()
    want = ozaki2.dgemm(a, b, 16)
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


def test_dgemm_strided_operands():
    announce("dgemm strided")
    a, b = ozk_inputs.gemm_operands(50, 40, 77, seed=4)
    abig = np.zeros((50, 90))
    abig[:, :77] = a
    bbig = np.zeros((77, 45))
    bbig[:, :40] = b
    da, db = to_dev(abig)[:, :77], to_dev(bbig)[:, :40]
    out = torch.full((50, 48), 7.0, dtype=torch.float64, device=da.device)
    ozk.ozk_dgemm(da, db, 14, out=out[:, :40])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[:, 40:] == 7.0)
    assert assert_within_ulps(got[:, :40], ozaki2.dgemm(a, b, 14), 2) == 0


def test_dgemm_tiny_config_normwise():
    """64^3, U(-1,1), r = 14: normwise error <= 1e-15 against Dot2."""
    announce("dgemm tiny normwise")
    a, b = ozk_inputs.gemm_operands(64, 64, 64, seed=1, dist="uniform")
    got = ozk.ozk_dgemm(to_dev(a), to_dev(b), 14).cpu().numpy()
    dd = reference.dot2_matmul(a, b)
    assert np.linalg.norm(got - dd) / np.linalg.norm(dd) <= 1e-15


def test_dgemm_deterministic():
    announce("dgemm determinism")
    a, b = ozk_inputs.gemm_operands(300, 300, 300, seed=2, dist="phi", phi=0.5)
    da, db = to_dev(a), to_dev(b)
    c1 = ozk.ozk_dgemm(da, db, 16)
    c2 = ozk.ozk_dgemm(da, db, 16)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int64), c2.view(torch.int64))


@pytest.mark.parametrize("r", list(range(12, 19)))
def test_dgemm_square_4096_sampled(r):
    """The 4096^3 configuration, entries (U-0.5) exp(0.5 N), sampled outputs vs oracle."""
    announce(f"dgemm 4096^3 r={r} sampled")
    a, b = ozk_inputs.gemm_operands(4096, 4096, 4096, seed=2, dist="phi", phi=0.5)
    got = ozk.ozk_dgemm(to_dev(a), to_dev(b), r)
    torch.cuda.synchronize()
    rng = np.random.default_rng(r)
    rows = np.sort(rng.choice(4096, 12, replace=False))
    cols = np.sort(rng.choice(4096, 40, replace=False))
    rows[-1], cols[-1] = 4095, 4095
    want = ozaki2.dgemm(a, b, r, rows=rows, cols=cols)
    sub = got[torch.as_tensor(rows, device=got.device)][:, torch.as_tensor(cols, device=got.device)]
    assert assert_within_ulps(sub.cpu().numpy(), want, 2) == 0


def test_dgemm_4096_error_vs_r():
    """The 4096^3 workload's output error against the exact product, on a sampled block,
    as r sweeps 12..18: it falls with every added modulus and reaches normwise 1e-15 at
    r = 16 (the configuration the benchmark times)."""
    announce("dgemm 4096^3 error vs r")
    a, b = ozk_inputs.gemm_operands(4096, 4096, 4096, seed=2, dist="phi", phi=0.5)
    da, db = to_dev(a), to_dev(b)
    rng = np.random.default_rng(11)
    rows = np.sort(rng.choice(4096, 6, replace=False))
    cols = np.sort(rng.choice(4096, 48, replace=False))
    exact = reference.exact_matmul(a[rows], b[:, cols])
    r_i = torch.as_tensor(rows, device=da.device)
    c_i = torch.as_tensor(cols, device=da.device)
    errs = {}
    for r in range(12, 19):
        got = ozk.ozk_dgemm(da, db, r)[r_i][:, c_i].cpu().numpy()
        errs[r] = float(np.linalg.norm(got - exact) / np.linalg.norm(exact))
    announce(f"errors {errs}")
    assert errs[16] <= 1e-15
    assert errs[12] > 1e-13
    for r in range(12, 16):
        assert errs[r + 1] < errs[r] / 4


def test_modular_products_at_the_int32_bound():
    """kp = 131072 (the largest K the planes allow) with every term (-128)(-128) except
    one zero K column: the sum 131071 * 2^14 = 2^31 - 2^14 is the largest an int32 must
    hold exactly, through the whole-line (pair-stage) product kernel."""
    announce("modular products at the int32 bound")
    kp, m, n = 131072, 64, 96
    pa = np.full((1, m, kp), -128, dtype=np.int8)
    pb = np.full((1, n, kp), -128, dtype=np.int8)
    pa[:, :, -1] = 0
    pb[:, 5, :] = 127                     # a column with the other sign
    pb[:, 5, -1] = 0
    got = ozk.ozk_modular_products(to_dev(pa), to_dev(pb)).cpu().numpy().astype(np.int64)
    want = ozaki2.modular_products(pa, pb)
    np.testing.assert_array_equal(got, want)
    assert want[0, 0, 0] == 131071 * 2**14 and want[0, 0, 5] == -131071 * 128 * 127
    got_r = ozk.ozk_modular_residues(to_dev(pa), to_dev(pb), r=1).cpu().numpy()
    np.testing.assert_array_equal(got_r.astype(np.int64), ((want + 128) % 256) - 128)


@pytest.mark.parametrize("scaling", ["max", "norm"])
def test_dgemm_largest_k(scaling):
    """k = 131071, the largest inner dimension: row deconstruction by the two-pass path,
    K padded to 131072, against the oracle (norm rule: fed the GPU exponents)."""
    announce(f"dgemm k=131071 {scaling}")
    m, n, k, r = 24, 40, 131071, 16
    a, b = ozk_inputs.gemm_operands(m, n, k, seed=17, dist="phi", phi=1.0)
    got = ozk.ozk_dgemm_ex(to_dev(a), to_dev(b), r, scaling).cpu().numpy()
    if scaling == "max":
        want = ozaki2.dgemm(a, b, r)
    else:
        _, e = ozk.ozk_deconstruct_ex(to_dev(a), 0, r, "norm", k_budget=k)
        _, f = ozk.ozk_deconstruct_ex(to_dev(b), 1, r, "norm", k_budget=k)
        want = ozaki2.dgemm(a, b, r, exps=(e.cpu().numpy().astype(np.int64),
                                          f.cpu().numpy().astype(np.int64)))
    assert assert_within_ulps(got, want, 2) == 0


def test_dgemm_timed_equals_untimed():
    """ozk_dgemm_ex_timed: the same result as ozk_dgemm_ex, bit for bit, and its events
    bracket the residue products (a positive time below the whole call's)."""
    announce("dgemm timed entry point")
    a, b = ozk_inputs.gemm_operands(600, 520, 700, seed=17, dist="phi", phi=2.0)
    da, db = to_dev(a), to_dev(b)
    plain = ozk.ozk_dgemm_ex(da, db, 16, "max")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    ev[0].record()
    timed = ozk.ozk_dgemm_ex_timed(da, db, 16, ev[1], ev[2], "max")
    ev[3].record()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(timed.cpu().numpy(), plain.cpu().numpy())
    inner, outer = ev[1].elapsed_time(ev[2]), ev[0].elapsed_time(ev[3])
    assert 0.0 < inner <= outer
    want = ozaki2.dgemm(a, b, 16)
    assert assert_within_ulps(timed.cpu().numpy(), want, 2) == 0
