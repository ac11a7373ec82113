"""C-ABI checks that need no GPU: the library loads, exports every function the header
declares, reports the documented constants, and rejects bad arguments before any HIP
call."""
import ctypes
import os
import re

import pytest

import fp64_gemm_emulation_ozk_amd as ozk
from oracle import rns

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ozk.h")

OK, EINVAL, EWORKSPACE, ERANGE, EHIP, EUNSUPPORTED = 0, -1, -2, -3, -4, -5


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ozk.LIB_PATH):
        from fp64_gemm_emulation_ozk_amd.build import build_library
        build_library(verbose=False)
    return ozk.library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ozk_[a-z0-9_]+)\s*\(", text)))


def test_header_functions_exported(lib):
    names = _declared_functions()
    assert len(names) >= 17
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(ozk._SIGNATURES), "binding and header declare different functions"


def test_version_and_status_strings(lib):
    assert lib.ozk_version() >= 100
    for st in (OK, EINVAL, EWORKSPACE, ERANGE, EHIP, EUNSUPPORTED, 12345):
        assert isinstance(lib.ozk_status_string(st), bytes)


@pytest.mark.parametrize("r", [1, 7, 14, 20])
def test_moduli_match_oracle(lib, r):
    assert ozk.ozk_moduli(r) == rns.moduli(r)


def test_moduli_rejects_bad_r(lib):
    buf = (ctypes.c_int32 * 21)()
    assert lib.ozk_moduli(0, ctypes.cast(buf, ctypes.c_void_p)) == EINVAL
    assert lib.ozk_moduli(21, ctypes.cast(buf, ctypes.c_void_p)) == EINVAL
    assert lib.ozk_moduli(3, None) == EINVAL


@pytest.mark.parametrize("r,k", [(14, 64), (12, 4096), (16, 4096), (18, 4096), (20, 8192),
                                 (14, 32768), (5, 100), (16, 131071),
                                 # the 76-bit cap: r = 20 with k = 1 and 2 (beta 154, 153)
                                 (20, 1), (20, 2), (20, 3), (19, 1)])
def test_scaling_bits_match_oracle(lib, r, k):
    assert ozk.ozk_scaling_bits(r, k) == rns.scaling_bits(r, k)


def test_scaling_bits_errors(lib):
    pa, pb = ctypes.c_int32(), ctypes.c_int32()
    assert lib.ozk_scaling_bits(16, 131072, ctypes.byref(pa), ctypes.byref(pb)) == ERANGE
    assert lib.ozk_scaling_bits(1, 64, ctypes.byref(pa), ctypes.byref(pb)) == ERANGE
    assert lib.ozk_scaling_bits(0, 64, ctypes.byref(pa), ctypes.byref(pb)) == EINVAL
    assert lib.ozk_scaling_bits(5, 0, ctypes.byref(pa), ctypes.byref(pb)) == EINVAL


@pytest.mark.parametrize("r,k", [(2, 1), (3, 64), (8, 4096), (12, 4096), (16, 4096),
                                 (18, 4096), (20, 8192), (14, 32768), (16, 131071)])
def test_scaling_bits_ex_match_oracle(lib, r, k):
    assert ozk.ozk_scaling_bits_ex(r, k, "max") == rns.scaling_bits(r, k)
    assert ozk.ozk_scaling_bits_ex(r, k, "norm") == rns.scaling_bits_norm(r, k)


def test_scaling_bits_ex_errors(lib):
    pa, pb = ctypes.c_int32(), ctypes.c_int32()
    f = lib.ozk_scaling_bits_ex
    assert f(16, 4096, 2, ctypes.byref(pa), ctypes.byref(pb)) == EINVAL       # unknown rule
    assert f(16, 4096, -1, ctypes.byref(pa), ctypes.byref(pb)) == EINVAL
    assert f(16, 131072, 1, ctypes.byref(pa), ctypes.byref(pb)) == ERANGE     # k too large
    assert f(0, 64, 1, ctypes.byref(pa), ctypes.byref(pb)) == EINVAL
    with pytest.raises(ValueError):
        rns.scaling_bits_norm(1, 1 << 16)
    assert f(1, 1 << 16, 1, ctypes.byref(pa), ctypes.byref(pb)) == ERANGE     # no budget


def test_planes_ld(lib):
    assert [lib.ozk_planes_ld(k) for k in (1, 63, 64, 65, 4096, 4097)] == [64, 64, 64, 128, 4096,
                                                                          4160]


def test_workspace_sizes(lib):
    ws = ozk.ozk_dgemm_workspace_size(4096, 4096, 4096, 16)
    assert ws >= 16 * 4096 * 4096 * 3           # two operand plane sets + residues
    out = ctypes.c_size_t()
    assert lib.ozk_dgemm_workspace_size(4, 4, 200000, 16, ctypes.byref(out)) == ERANGE
    assert lib.ozk_dgemm_workspace_size(4, 4, 4, 0, ctypes.byref(out)) == EINVAL
    # one query serves both rules: the norm rule's chunk partials (a maximum and a sum per
    # 128 rows of a column; per 2048 columns of a row the fused kernel cannot hold)
    assert ozk.ozk_deconstruct_workspace_size(4096, 4096, 1) >= 2 * 32 * 4096 * 8
    assert ozk.ozk_deconstruct_workspace_size(4096, 4096, 0) == 0
    assert ozk.ozk_deconstruct_workspace_size(8, 40000, 0) >= 2 * 8 * 20 * 8
    assert ws >= 16 * 4096 * 4096 * 3 + 2 * 32 * 4096 * 8


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def test_dgemm_validation_before_any_hip_call(lib):
    f = lib.ozk_dgemm
    assert f(4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 0, FAKE, 1 << 20, None) == EINVAL   # r
    assert f(4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 21, FAKE, 1 << 20, None) == EINVAL  # r
    assert f(4, 4, 200000, FAKE, 200000, FAKE, 4, FAKE, 4, 16, FAKE, 1 << 20, None) == ERANGE
    assert f(4, 4, 4, FAKE, 3, FAKE, 4, FAKE, 4, 14, FAKE, 1 << 20, None) == EINVAL  # lda < k
    assert f(4, 4, 4, FAKE, 4, FAKE, 3, FAKE, 4, 14, FAKE, 1 << 20, None) == EINVAL  # ldb < n
    assert f(4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 3, 14, FAKE, 1 << 20, None) == EINVAL  # ldc < n
    assert f(-1, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 14, FAKE, 1 << 20, None) == EINVAL
    assert f(4, 4, 4, None, 4, FAKE, 4, FAKE, 4, 14, FAKE, 1 << 20, None) == EINVAL  # null A
    assert f(4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 14, None, 0, None) == EWORKSPACE
    assert f(4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 14, FAKE, 16, None) == EWORKSPACE
    assert f(4, 4, 1 << 16, FAKE, 1 << 16, FAKE, 4, FAKE, 4, 2, FAKE, 1 << 30, None) == ERANGE
    assert f(0, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 14, None, 0, None) == OK           # empty


def test_deconstruct_validation(lib):
    f = lib.ozk_deconstruct
    # ldp not a multiple of 64, ldp < K, bad axis, bad r, short plane stride, null planes
    assert f(FAKE, 4, 100, 100, 0, 14, 100, FAKE, 100, 400, FAKE, FAKE, 0, None) == EINVAL
    assert f(FAKE, 4, 100, 100, 0, 14, 100, FAKE, 64, 256, FAKE, FAKE, 0, None) == EINVAL
    assert f(FAKE, 4, 100, 100, 2, 14, 100, FAKE, 128, 512, FAKE, FAKE, 0, None) == EINVAL
    assert f(FAKE, 4, 100, 100, 0, 0, 100, FAKE, 128, 512, FAKE, FAKE, 0, None) == EINVAL
    assert f(FAKE, 4, 100, 100, 0, 14, 100, FAKE, 128, 256, FAKE, FAKE, 0, None) == EINVAL
    assert f(FAKE, 4, 100, 100, 0, 14, 100, None, 128, 512, FAKE, FAKE, 0, None) == EINVAL
    # axis 1 needs a column-maximum workspace
    assert f(FAKE, 100, 4, 4, 1, 14, 100, FAKE, 128, 512, FAKE, None, 0, None) == EWORKSPACE


def test_ex_validation(lib):
    f = lib.ozk_dgemm_ex
    assert f(4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 14, 2, FAKE, 1 << 20, None) == EINVAL  # rule
    assert f(4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 14, -1, FAKE, 1 << 20, None) == EINVAL
    assert f(4, 4, 4, FAKE, 3, FAKE, 4, FAKE, 4, 14, 1, FAKE, 1 << 20, None) == EINVAL   # lda
    assert f(4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 14, 1, None, 0, None) == EWORKSPACE
    assert f(4, 4, 1 << 16, FAKE, 1 << 16, FAKE, 4, FAKE, 4, 1, 1, FAKE, 1 << 30,
             None) == ERANGE                                                          # budget
    assert f(0, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 14, 1, None, 0, None) == OK           # empty
    g = lib.ozk_deconstruct_ex
    assert g(FAKE, 4, 100, 100, 0, 14, 100, 5, FAKE, 128, 512, FAKE, FAKE, 0, None) == EINVAL
    assert g(FAKE, 4, 100, 100, 0, 14, 100, 1, FAKE, 64, 256, FAKE, FAKE, 0, None) == EINVAL
    # axis 1 by the norm rule needs the chunk partials: missing, too small, misaligned
    assert g(FAKE, 100, 4, 4, 1, 14, 100, 1, FAKE, 128, 512, FAKE, None, 0, None) == EWORKSPACE
    assert g(FAKE, 100, 4, 4, 1, 14, 100, 1, FAKE, 128, 512, FAKE, FAKE, 8, None) == EWORKSPACE
    assert g(FAKE, 100, 4, 4, 1, 14, 100, 1, FAKE, 128, 512, FAKE, ctypes.c_void_p(0x1004),
             1 << 20, None) == EINVAL


def test_dgemm_timed_validation(lib):
    f = lib.ozk_dgemm_ex_timed
    # one event without the other
    assert f(4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 14, 1, FAKE, 1 << 20, None, FAKE,
             None) == EINVAL
    assert f(4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 14, 1, FAKE, 1 << 20, None, None,
             FAKE) == EINVAL
    # otherwise the checks of ozk_dgemm_ex
    assert f(4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 14, 2, FAKE, 1 << 20, None, None,
             None) == EINVAL
    assert f(0, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 14, 1, None, 0, None, None, None) == OK


def test_spmv_validation(lib):
    f = lib.ozk_spmv_csr
    out = ctypes.c_size_t()
    assert lib.ozk_spmv_csr_workspace_size(10, 0, 14, ctypes.byref(out)) == EINVAL
    assert lib.ozk_spmv_csr_workspace_size(10, 10, 14, ctypes.byref(out)) == OK
    assert out.value >= 14 * 10 + 10 * 4 + 10 * 16     # row sums, row exponents, x residues
    args = lambda **kw: dict(dict(rows=10, cols=10, nnz=30, kmax=7, r=14, ws=FAKE, wsb=1 << 20),
                             **kw)
    call = lambda a: f(a["rows"], a["cols"], a["nnz"], FAKE, FAKE, FAKE, a["kmax"], FAKE, FAKE,
                       a["r"], a["ws"], a["wsb"], None)
    assert call(args(r=0)) == EINVAL
    assert call(args(cols=0)) == EINVAL
    assert call(args(kmax=0)) == EINVAL
    assert call(args(nnz=-1)) == EINVAL
    assert call(args(kmax=131072)) == ERANGE
    assert call(args(r=1, kmax=1000)) == ERANGE          # no bit budget
    assert call(args(ws=None, wsb=0)) == EWORKSPACE
    assert call(args(wsb=16)) == EWORKSPACE
    assert call(args(nnz=1 << 31)) == EUNSUPPORTED
    assert call(args(rows=0, ws=None, wsb=0)) == OK      # nothing to do


def test_products_and_reconstruct_validation(lib):
    f = lib.ozk_modular_products
    assert f(4, 4, 100, 3, FAKE, 400, FAKE, 400, FAKE, 4, 16, None) == EINVAL       # kp % 64
    assert f(4, 4, 64, 3, FAKE, 128, FAKE, 256, FAKE, 4, 16, None) == EINVAL        # stride_a
    assert f(4, 4, 131136, 3, FAKE, 1 << 20, FAKE, 1 << 20, FAKE, 4, 16, None) == ERANGE
    g = lib.ozk_reconstruct
    assert g(4, 4, 0, FAKE, 4, 16, FAKE, FAKE, FAKE, 4, None) == EINVAL
    assert g(4, 4, 3, FAKE, 3, 16, FAKE, FAKE, FAKE, 4, None) == EINVAL             # ld < n
    assert g(4, 4, 3, None, 4, 16, FAKE, FAKE, FAKE, 4, None) == EINVAL


def test_no_measurement_probe_exported(lib):
    """The library exports the method's entry points only (no matrix-core rate probe)."""
    assert not hasattr(lib, "ozk_probe_mfma")


def test_noalloc_gemv_validation(lib):
    """ozk_dgemv_noalloc checks its arguments like ozk_dgemv and refuses a request whose
    scratch exceeds its fixed array (OZK_ENOSCRATCH = -6), all before any HIP call."""
    f = lib.ozk_dgemv_noalloc
    assert f(64, 64, 33, FAKE, 64, None, 0, 0, None, FAKE, 33, FAKE, 33, 14, 0, None) == EINVAL
    assert f(64, 64, 2, FAKE, 64, None, 0, 0, None, FAKE, 2, FAKE, 2, 21, 0, None) == EINVAL
    assert f(64, 64, 2, None, 64, None, 0, 0, None, FAKE, 2, FAKE, 2, 14, 0, None) == EINVAL
    assert f(64, 1 << 17, 2, FAKE, 1 << 17, None, 0, 0, None, FAKE, 2, FAKE, 2, 14, 0,
             None) == ERANGE
    assert f(0, 64, 2, None, 64, None, 0, 0, None, None, 2, None, 2, 14, 0, None) == OK
    need = ozk.ozk_dgemv_workspace_size(32768, 32768, 16, 14, 0)
    assert need > ozk.OZK_NOALLOC_SCRATCH_BYTES
    assert f(32768, 32768, 16, FAKE, 32768, None, 0, 0, None, FAKE, 16, FAKE, 16, 14, 0,
             None) == -6
    assert ozk.ozk_dgemv_workspace_size(32768, 32768, 32, 14, 0) <= ozk.OZK_NOALLOC_SCRATCH_BYTES
    assert b"scratch" in lib.ozk_status_string(-6)
