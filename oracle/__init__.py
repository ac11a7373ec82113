"""CPU oracle for Ozaki-scheme-II fp64 GEMM/GEMV emulation and the FP4-limb INT8 product.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code, tables or constant generators with the HIP
library; the two meet only through the seeded generators in ``ozk_inputs``.

Sources it follows (cited by page title and part):

* [TME4] "The Missing Fourth Term for the Emulation Tensor Memory Equilibrium (TME)
  Model: The Residue Deconstruction Cost", arXiv 2610.10924v1, abstract: emulation of
  fp64 by Ozaki scheme II, in which every fp64 operand is scaled, rounded and reduced
  modulo each of r moduli before the integer matrix products, and a per-output
  reconstruction returns fp64; storing the residues moves that cost into HBM traffic.
* [AWE] arXiv 2609.24519 listing (Nagoya University), English abstract: each Ozaki
  product is an exact integer matrix product times a scale; the set S of FP4 values
  times 2 holds every residue modulo 13, so integers split into base-13 digits with
  weights (1, 13, 169), and an INT8 x INT8 product takes 9 pairwise FP4 GEMMs; with
  free limb weights and planes that combine limbs it takes 6, and INT4 x INT8 takes 4.

Where the pages leave a step open, the module that implements it states the reading it
takes (moduli, scaling rule, symmetric range, digit choice, e2m1 nibble order).

Modules:
    rns        moduli, CRT basis, bit budgets, symmetric residue, CRT lift (Python ints)
    ozaki2     exponents, scaled integers, residue planes, modular products, reconstruction
    reference  Dot2 double-double dot products and exact rational products (accuracy pins)
    fp4limb    base-13 digit split, e2m1 codes, 9-product limb GEMM
    fp4awe     weights (1, 29, 37), limb and pairwise-sum planes, 6-product limb GEMM
    fp4awe4    INT4 x INT8 in 4 FP4 products (limb weight 5, planes at four points)
    spmv       emulated CSR sparse matrix-vector product
"""
from . import rns, ozaki2, reference, fp4limb, fp4awe, spmv  # noqa: F401
