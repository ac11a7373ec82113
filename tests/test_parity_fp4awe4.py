"""GPU parity of the exact INT4 x INT8 product in 4 FP4 plane products (limb weight 5,
planes at the points 0, inf, 1, 1/2, coefficients 36, 90, 45, -10).

Packed planes, the 4 plane products and the combined int32 result must all be bit-exact
against the oracle (oracle/fp4awe4.py) and the exact integer product."""
import numpy as np
import pytest
import torch

import fp64_gemm_emulation_ozk_amd as ozk
import ozk_inputs
from oracle import fp4awe4

from gpu_common import announce, to_dev

pytestmark = pytest.mark.gpu


def _kpad(k):
    return (k + 63) // 64 * 64


def _planes(x, int4):
    return fp4awe4.planes_x(x) if int4 else fp4awe4.planes_y(x)


@pytest.mark.parametrize("rows,cols,axis", [(37, 100, 0), (5, 64, 0), (100, 37, 1),
                                            (300, 130, 1), (1, 1, 0), (1, 1, 1),
                                            (9, 208, 0), (33, 512, 0), (70, 64, 1),
                                            (45, 260, 1)])
@pytest.mark.parametrize("int4", [True, False])
def test_pack_bit_exact(rows, cols, axis, int4):
    announce(f"fp4awe4 pack rows={rows} cols={cols} axis={axis} int4={int4}")
    rng = np.random.default_rng(rows * 5 + cols + int4)
    x = ozk_inputs.int8_matrix(rng, (rows, cols))      # int4: only the low nibble counts
    x.flat[0] = -128
    x.flat[-1] = 127
    got = ozk.ozk_fp4awe4_pack(to_dev(x), axis, int4).cpu().numpy()
    src = x if axis == 0 else x.T
    want = fp4awe4.pack_lines(_planes(src, int4), _kpad(src.shape[1]))
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("int4", [True, False])
def test_pack_every_value(int4):
    announce(f"fp4awe4 pack all 256 bytes int4={int4}")
    x = np.arange(-128, 128, dtype=np.int8).reshape(2, 128)
    got = ozk.ozk_fp4awe4_pack(to_dev(x), 0, int4).cpu().numpy()
    np.testing.assert_array_equal(got, fp4awe4.pack_lines(_planes(x, int4), 128))


@pytest.mark.parametrize("m,n,k", [(33, 29, 70), (64, 96, 256), (130, 70, 1000), (1, 1, 1)])
def test_plane_products_bit_exact(m, n, k):
    announce(f"fp4awe4 4 products m={m} n={n} k={k}")
    a, b = ozk_inputs.int4_int8_operands(m, n, k, seed=m + 2 * n + k)
    pa = ozk.ozk_fp4awe4_pack(to_dev(a), 0, True)
    pb = ozk.ozk_fp4awe4_pack(to_dev(b), 1, False)
    got = ozk.ozk_fp4awe4_products(pa, pb, k).cpu().numpy()
    np.testing.assert_array_equal(got.astype(np.int64), fp4awe4.plane_products(a, b))


def _exact(a, b):
    return a.astype(np.int64) @ b.astype(np.int64)


# tiles of 128 x 128: one partial tile, several tiles with ragged edges, K not a multiple
# of 64, one K step, more steps than the 3-stage ring, odd and even step counts
@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (33, 29, 70), (128, 128, 64), (300, 257, 129),
                                   (257, 520, 1000), (64, 40, 8192), (129, 130, 192),
                                   (400, 384, 3 * 64), (128, 256, 4 * 64)])
def test_int4int8gemm_fp4awe_exact(m, n, k):
    announce(f"fp4awe4 gemm m={m} n={n} k={k}")
    a, b = ozk_inputs.int4_int8_operands(m, n, k, seed=11 * m + n + k)
    got = ozk.ozk_int4int8gemm_fp4awe(to_dev(a), to_dev(b)).cpu().numpy()
    np.testing.assert_array_equal(got.astype(np.int64), _exact(a, b))


def test_int4int8gemm_fp4awe_reads_low_nibble():
    """A holds arbitrary bytes; the product is that of their low nibbles as int4."""
    announce("fp4awe4 gemm low nibble")
    rng = np.random.default_rng(8)
    a = ozk_inputs.int8_matrix(rng, (70, 300))
    b = ozk_inputs.int8_matrix(rng, (300, 50))
    vals = ((a.astype(np.int64) & 15) ^ 8) - 8
    got = ozk.ozk_int4int8gemm_fp4awe(to_dev(a), to_dev(b)).cpu().numpy()
    np.testing.assert_array_equal(got.astype(np.int64), vals @ b.astype(np.int64))
    np.testing.assert_array_equal(got.astype(np.int64), fp4awe4.int4_int8_gemm(a, b))


def _largest_plane_value(table, planes):
    return max(table, key=lambda v: sum(abs(t) for t in planes(table[v])))


# (-7, -105): the pair whose shared sum 2 P1 + P2 is largest (27 per K value)
@pytest.mark.parametrize("va,vb", [(-8, -128), (7, -128), (-8, 127), ("big", "big"),
                                   (-7, -105)])
def test_int4int8gemm_fp4awe_accumulator_bound(va, vb):
    """Constant operands with K = 131071 (the largest K): every plane product sums K equal
    terms of up to 48 in magnitude, 6.3 M, and the shared sum 2 P1 + P2 terms of up to 27,
    3.5 M, still integers below 2^24 in fp32."""
    if va == "big":
        va = _largest_plane_value(fp4awe4.x_table(), fp4awe4.x_planes)
        vb = _largest_plane_value(fp4awe4.y_table(), fp4awe4.y_planes)
    k = 131071
    announce(f"fp4awe4 gemm bound k={k} va={va} vb={vb}")
    a = np.full((40, k), va, dtype=np.int8)
    b = np.full((k, 36), vb, dtype=np.int8)
    a[3, 5] = 0
    got = ozk.ozk_int4int8gemm_fp4awe(to_dev(a), to_dev(b)).cpu().numpy()
    np.testing.assert_array_equal(got.astype(np.int64), _exact(a, b))


def test_int4int8gemm_fp4awe_strided():
    announce("fp4awe4 gemm strided")
    a, b = ozk_inputs.int4_int8_operands(50, 40, 77, seed=4)
    abig = np.zeros((50, 96), np.int8)
    abig[:, :77] = a
    bbig = np.zeros((77, 48), np.int8)
    bbig[:, :40] = b
    out = torch.full((50, 44), 9, dtype=torch.int32, device="cuda")
    ozk.ozk_int4int8gemm_fp4awe(to_dev(abig)[:, :77], to_dev(bbig)[:, :40], out=out[:, :40])
    got = out.cpu().numpy()
    assert np.all(got[:, 40:] == 9)
    np.testing.assert_array_equal(got[:, :40].astype(np.int64), _exact(a, b))


def test_int4int8gemm_fp4awe_equals_six_product_engine():
    """On int4-valued A the 4-product and 6-product engines give the same bits."""
    announce("fp4awe4 equals the 6-product engine")
    a, b = ozk_inputs.int4_int8_operands(700, 650, 2000, seed=21)
    da, db = to_dev(a), to_dev(b)
    four = ozk.ozk_int4int8gemm_fp4awe(da, db)
    six = ozk.ozk_int8gemm_fp4awe(da, db)
    torch.cuda.synchronize()
    assert torch.equal(four, six)


def test_int4int8gemm_fp4awe_8192_full():
    """8192^3 (A int4 uniform in [-8, 7], B int8 uniform in [-128, 127], seed 5): every
    output against the exact product in float64 BLAS on the host (exact: |partial sums|
    <= 2^23 < 2^53); a second call gives the same bits."""
    announce("fp4awe4 gemm 8192^3 full output")
    a, b = ozk_inputs.int4_int8_operands(8192, 8192, 8192, seed=5)
    da, db = to_dev(a), to_dev(b)
    got = ozk.ozk_int4int8gemm_fp4awe(da, db)
    again = ozk.ozk_int4int8gemm_fp4awe(da, db)
    torch.cuda.synchronize()
    assert torch.equal(got, again)
    want = a.astype(np.float64) @ b.astype(np.float64)
    np.testing.assert_array_equal(got.cpu().numpy(), want.astype(np.int32))
