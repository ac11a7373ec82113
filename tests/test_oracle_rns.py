"""Pins for oracle.rns: moduli, CRT basis, bit budgets, symmetric residues.

Each check is against a closed form or brute force, never against the oracle's own
formula retyped."""
import math
import random
from fractions import Fraction

import pytest

from oracle import rns


def test_moduli_pairwise_coprime_and_bounded():
    ms = rns.moduli(20)
    assert len(ms) == 20 and len(set(ms)) == 20
    assert all(2 <= m <= 256 for m in ms)
    for i in range(20):
        for j in range(i + 1, 20):
            assert math.gcd(ms[i], ms[j]) == 1


def test_moduli_greedy_maximal():
    """Every integer above the smallest chosen modulus that was skipped shares a factor
    with a larger chosen one (so no larger coprime candidate was passed over), and the
    list is strictly decreasing: the greedy reading, checked by brute force."""
    ms = rns.moduli(20)
    assert ms == sorted(ms, reverse=True)
    chosen = set(ms)
    for c in range(ms[-1], 257):
        if c in chosen:
            continue
        larger = [m for m in ms if m > c]
        assert any(math.gcd(c, m) > 1 for m in larger), c


def test_moduli_prefix_property():
    for r in range(1, 21):
        assert rns.moduli(r) == rns.moduli(20)[:r]
    with pytest.raises(ValueError):
        rns.moduli(0)
    with pytest.raises(ValueError):
        rns.moduli(21)


@pytest.mark.parametrize("r", [1, 2, 5, 12, 14, 16, 18, 20])
def test_crt_basis_kronecker(r):
    big_m, basis = rns.crt_basis(r)
    ms = rns.moduli(r)
    assert big_m == math.prod(ms)
    for l, e in enumerate(basis):
        assert 0 < e < big_m
        for j, m in enumerate(ms):
            assert e % m == (1 if j == l else 0)


@pytest.mark.parametrize("r", [3, 14, 20])
def test_crt_lift_roundtrip(r):
    big_m, _ = rns.crt_basis(r)
    ms = rns.moduli(r)
    rng = random.Random(r)
    half = (big_m - 1) // 2
    samples = [0, 1, -1, half, -half] + [rng.randint(-half, half) for _ in range(300)]
    for x in samples:
        res = [x % m for m in ms]
        assert rns.crt_lift(res, r) == x
        sres = [rns.smod(x, m) for m in ms]
        assert rns.crt_lift(sres, r) == x


@pytest.mark.parametrize("r", range(1, 21))
def test_budget_q_is_floor_log2(r):
    big_m, _ = rns.crt_basis(r)
    q = rns.budget_q(r)
    assert 2**q <= (big_m - 1) // 2 < 2 ** (q + 1)


@pytest.mark.parametrize("r,k", [(14, 64), (12, 4096), (16, 4096), (18, 4096), (16, 8192),
                                 (20, 8192), (14, 32768), (20, 1), (8, 100), (16, 4097)])
def test_scaling_bits_guarantee_exact_crt(r, k):
    """k 2^PA 2^PB <= (M-1)/2 (exact recovery) and the budget is tight: one more bit
    would break the power-of-two bound at the next power of two of k."""
    big_m, _ = rns.crt_basis(r)
    pa, pb = rns.scaling_bits(r, k)
    assert pa <= pb <= pa + 1
    assert k * 2 ** (pa + pb) <= (big_m - 1) // 2
    kk = 1 << rns.ceil_log2(k)
    assert kk >= k and (kk == 1 or kk // 2 < k)
    if pb < rns.WIDTH_CAP:
        assert kk * 2 ** (pa + pb + 1) > 2 ** rns.budget_q(r)


@pytest.mark.parametrize("r", range(1, 21))
@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 64])
def test_scaling_bits_capped_at_76(r, k):
    """Every width stays at or below 76 bits; the cap binds only at r = 20 with k <= 2,
    where beta = Q - ceil(log2 k) is 154 or 153 (widths (76, 76) instead of (77, 77) and
    (76, 77)); everywhere else the widths are floor(beta/2) and beta - floor(beta/2)."""
    try:
        pa, pb = rns.scaling_bits(r, k)
    except ValueError:
        return
    beta = rns.budget_q(r) - rns.ceil_log2(k)
    assert max(pa, pb) <= 76
    if r == 20 and k <= 2:
        assert (pa, pb) == (76, 76) and beta in (153, 154)
    else:
        assert (pa, pb) == (beta // 2, beta - beta // 2)


def test_scaling_bits_no_budget():
    with pytest.raises(ValueError):
        rns.scaling_bits(1, 1 << 20)


@pytest.mark.parametrize("m", [2, 3, 13, 173, 217, 255, 256])
def test_smod_exhaustive(m):
    lo, hi = -(m // 2), (m + 1) // 2 - 1
    seen = set()
    for x in range(-5 * m - 3, 5 * m + 4):
        s = rns.smod(x, m)
        assert lo <= s <= hi
        assert (x - s) % m == 0
        seen.add(s)
    assert seen == set(range(lo, hi + 1))
    assert rns.smod(128, 256) == -128 and rns.smod(127, 256) == 127


@pytest.mark.parametrize("r", [1, 2, 3, 5, 8, 12, 14, 16, 18, 19, 20])
@pytest.mark.parametrize("k", [1, 2, 63, 64, 4096, 32768, 131071])
def test_norm_budget_exact_and_maximal(r, k):
    """(alpha_A, alpha_B) satisfy (2^aA + sqrt(k)/2)(2^aB + sqrt(k)/2) <= (M-1)/2 checked
    with exact rationals, and raising either width (within the cap and Q - 1) breaks it."""
    big_m, _ = rns.crt_basis(r)
    q = rns.budget_q(r)
    try:
        aa, ab = rns.scaling_bits_norm(r, k)
    except ValueError:
        # no budget: even (1, 1) fails the exact inequality
        assert not rns.norm_bound_holds(1, 1, k, big_m)
        return
    root_k = Fraction(math.isqrt(k)) if math.isqrt(k) ** 2 == k else None

    def exact_ok(x, y):
        # compare (2^x + s)(2^y + s) with (M-1)/2 for s = sqrt(k)/2, exactly: expand the
        # product; the sqrt(k) term is bounded by rationals from above when k is not a square
        s2 = Fraction(k, 4)
        lhs_rational = Fraction(2) ** (x + y) + s2
        coef = Fraction(2) ** x + Fraction(2) ** y          # multiplies sqrt(k)/2
        rhs = Fraction(big_m - 1, 2)
        if root_k is not None:
            return lhs_rational + coef * root_k / 2 <= rhs
        upper = Fraction(math.isqrt(k) + 1)                  # > sqrt(k)
        lower = Fraction(math.isqrt(k))                      # < sqrt(k)
        if lhs_rational + coef * upper / 2 <= rhs:
            return True
        if lhs_rational + coef * lower / 2 > rhs:
            return False
        return (rhs - lhs_rational) ** 2 * 4 >= coef ** 2 * k  # exact squared comparison
    assert exact_ok(aa, ab)
    assert aa + ab <= q - 1 and aa <= rns.NORM_ALPHA_CAP and ab <= rns.NORM_ALPHA_CAP
    for x, y in ((aa + 1, ab), (aa, ab + 1)):
        if x + y <= q - 1 and max(x, y) <= rns.NORM_ALPHA_CAP:
            assert not rns.norm_bound_holds(x, y, k, big_m)


def test_norm_budget_never_below_max_rule():
    for r in range(2, 21):
        for k in (64, 4096, 8192, 32768):
            try:
                pa, pb = rns.scaling_bits(r, k)
            except ValueError:
                continue
            aa, ab = rns.scaling_bits_norm(r, k)
            # a row with every |entry| equal makes ||a'||_2 = sqrt(k) max|a'|: the norm rule
            # then keeps floor(aA - log2 sqrt k) bits, no fewer than the max rule's P_A - 1
            assert aa + ab >= pa + pb
