"""Pins for oracle.rns: moduli, CRT basis, bit budgets, symmetric residues.

Each check is against a closed form or brute force, never against the oracle's own
formula retyped."""
import math
import random

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
    assert kk * 2 ** (pa + pb + 1) > 2 ** rns.budget_q(r)


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
