"""Pins for oracle.reference: Dot2 against the exact rational product and its
published error bound, and the exact product against hand-made cases."""
from fractions import Fraction

import numpy as np
import pytest

import ozk_inputs
from oracle import reference

U = 2.0**-53


def test_exact_matmul_hand_cases():
    a = np.array([[1.0, 2.0**-60], [3.0, -3.0]])
    b = np.array([[1.0, 0.1], [1.0, 0.1]])
    c = reference.exact_matmul(a, b)
    assert c[0, 0] == 1.0                  # 1 + 2^-60 rounds to 1
    assert c[1, 0] == 0.0 and c[1, 1] == 0.0
    s = reference.exact_matmul_ints(a, b)
    assert s[0, 0] == (1 << 2148) + (1 << (2148 - 60))


@pytest.mark.parametrize("dist,phi", [("uniform", 0.0), ("phi", 4.0)])
def test_dot2_error_bound(dist, phi):
    """Ogita-Rump-Oishi: |Dot2 - x.y| <= u |x.y| + gamma_k^2 sum |x_i y_i|."""
    a, b = ozk_inputs.gemm_operands(6, 5, 50, seed=4, dist=dist, phi=phi)
    got = reference.dot2_matmul(a, b)
    s = reference.exact_matmul_ints(a, b)
    k = a.shape[1]
    gamma = k * U / (1 - k * U)
    absdot = np.abs(a) @ np.abs(b)
    for i in range(6):
        for j in range(5):
            exact = int(s[i, j])
            e = abs(Fraction(got[i, j]) - Fraction(exact, 1 << 2148))
            bound = U * abs(Fraction(exact, 1 << 2148)) + Fraction(gamma**2 * absdot[i, j] * 1.01)
            assert e <= bound


def test_dot2_beats_plain_fp64_on_cancellation():
    x = np.array([[1e16, 1.0, -1e16, 1.0]])
    y = np.array([[1.0], [1.0], [1.0], [1.0]])
    assert reference.dot2_matmul(x, y)[0, 0] == 2.0
