"""Python binding of libozk.so (Ozaki-II fp64 GEMM/GEMV emulation and FP4-limb INT8
GEMM for MI355X).

Argument marshalling only: each ``ozk_*`` function here checks tensor devices, dtypes and
strides, allocates outputs and workspace with torch (device memory), and calls the C
entry point of the same name on the given stream (torch's current HIP stream by
default).  Every step of the
computation runs in the library's HIP kernels; there is no other code path.  If the
library is not built, loading fails with an error.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LIB_PATH", "OzkError", "library",
    "ozk_version", "ozk_moduli", "ozk_scaling_bits", "ozk_scaling_bits_ex", "ozk_planes_ld",
    "ozk_deconstruct", "ozk_deconstruct_ex", "ozk_modular_products", "ozk_modular_residues",
    "ozk_reconstruct", "ozk_dgemm", "ozk_dgemm_ex", "ozk_dgemm_ex_timed", "ozk_dgemv",
    "ozk_dgemv_noalloc", "OZK_NOALLOC_SCRATCH_BYTES",
    "ozk_spmv_csr",
    "ozk_spmv_csr_workspace_size",
    "OZK_SCALING_MAX", "OZK_SCALING_NORM",
    "ozk_fp4limb_pack", "ozk_fp4limb_products", "ozk_int8gemm_fp4limb",
    "ozk_fp4awe_line_bytes", "ozk_fp4awe_pack", "ozk_fp4awe_products", "ozk_int8gemm_fp4awe",
    "ozk_int8gemm_fp4awe_workspace_size",
    "ozk_fp4awe4_line_bytes", "ozk_fp4awe4_pack", "ozk_fp4awe4_products",
    "ozk_int4int8gemm_fp4awe", "ozk_int4int8gemm_fp4awe_workspace_size",
    "ozk_dgemm_workspace_size", "ozk_dgemv_workspace_size",
    "ozk_int8gemm_fp4limb_workspace_size", "ozk_deconstruct_workspace_size",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libozk.so")
OZK_PLANE_K = 64
OZK_NOALLOC_SCRATCH_BYTES = 64 << 20   # scratch array of ozk_dgemv_noalloc, per GPU

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_int = ctypes.c_int
_ptr = ctypes.c_void_p
_size = ctypes.c_size_t

_SIGNATURES = {
    "ozk_version": (_int, []),
    "ozk_status_string": (ctypes.c_char_p, [_int]),
    "ozk_moduli": (_int, [_int, _ptr]),
    "ozk_scaling_bits": (_int, [_int, _i64, _ptr, _ptr]),
    "ozk_scaling_bits_ex": (_int, [_int, _i64, _int, _ptr, _ptr]),
    "ozk_planes_ld": (_i64, [_i64]),
    "ozk_deconstruct_workspace_size": (_int, [_i64, _i64, _int, _ptr]),
    "ozk_deconstruct": (_int, [_ptr, _i64, _i64, _i64, _int, _int, _i64, _ptr, _i64, _i64, _ptr,
                               _ptr, _size, _ptr]),
    "ozk_modular_products": (_int, [_i64, _i64, _i64, _int, _ptr, _i64, _ptr, _i64, _ptr, _i64,
                                    _i64, _ptr]),
    "ozk_modular_residues": (_int, [_i64, _i64, _i64, _int, _ptr, _i64, _ptr, _i64, _ptr, _i64,
                                    _i64, _ptr]),
    "ozk_reconstruct": (_int, [_i64, _i64, _int, _ptr, _i64, _i64, _ptr, _ptr, _ptr, _i64, _ptr]),
    "ozk_deconstruct_ex": (_int, [_ptr, _i64, _i64, _i64, _int, _int, _i64, _int, _ptr, _i64,
                                  _i64, _ptr, _ptr, _size, _ptr]),
    "ozk_dgemm_ex": (_int, [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _int,
                            _ptr, _size, _ptr]),
    "ozk_dgemm_ex_timed": (_int, [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int,
                                  _int, _ptr, _size, _ptr, _ptr, _ptr]),
    "ozk_dgemm_workspace_size": (_int, [_i64, _i64, _i64, _int, _ptr]),
    "ozk_spmv_csr_workspace_size": (_int, [_i64, _i64, _int, _ptr]),
    "ozk_spmv_csr": (_int, [_i64, _i64, _i64, _ptr, _ptr, _ptr, _i64, _ptr, _ptr, _int, _ptr,
                            _size, _ptr]),
    "ozk_dgemm": (_int, [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _ptr, _size,
                         _ptr]),
    "ozk_dgemv_workspace_size": (_int, [_i64, _i64, _i64, _int, _int, _ptr]),
    "ozk_dgemv": (_int, [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _i64, _ptr, _ptr, _i64, _ptr,
                         _i64, _int, _int, _ptr, _size, _ptr]),
    "ozk_dgemv_noalloc": (_int, [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _i64, _ptr, _ptr, _i64,
                                 _ptr, _i64, _int, _int, _ptr]),
    "ozk_fp4limb_pack": (_int, [_ptr, _i64, _i64, _i64, _int, _ptr, _i64, _i64, _ptr]),
    "ozk_fp4limb_products": (_int, [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _i64,
                                    _ptr]),
    "ozk_int8gemm_fp4limb_workspace_size": (_int, [_i64, _i64, _i64, _ptr]),
    "ozk_fp4awe_line_bytes": (_i64, [_i64]),
    "ozk_fp4awe_pack": (_int, [_ptr, _i64, _i64, _i64, _int, _ptr, _i64, _ptr]),
    "ozk_fp4awe_products": (_int, [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _i64,
                                   _ptr]),
    "ozk_int8gemm_fp4awe_workspace_size": (_int, [_i64, _i64, _i64, _ptr]),
    "ozk_int8gemm_fp4awe": (_int, [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _ptr,
                                   _size, _ptr]),
    "ozk_int8gemm_fp4limb": (_int, [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _ptr,
                                    _size, _ptr]),
    "ozk_fp4awe4_line_bytes": (_i64, [_i64]),
    "ozk_fp4awe4_pack": (_int, [_ptr, _i64, _i64, _i64, _int, _int, _ptr, _i64, _ptr]),
    "ozk_fp4awe4_products": (_int, [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _i64,
                                    _ptr]),
    "ozk_int4int8gemm_fp4awe_workspace_size": (_int, [_i64, _i64, _i64, _ptr]),
    "ozk_int4int8gemm_fp4awe": (_int, [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _ptr,
                                       _size, _ptr]),
}

_LIB = None

OZK_SCALING_MAX = 0   # per-line maximum (the default of every entry point)
OZK_SCALING_NORM = 1  # per-line 2-norm (Cauchy-Schwarz)


def _scaling(scaling) -> int:
    names = {"max": OZK_SCALING_MAX, "norm": OZK_SCALING_NORM}
    if isinstance(scaling, str):
        if scaling not in names:
            raise ValueError(f"unknown scaling rule {scaling!r}")
        return names[scaling]
    return int(scaling)


class OzkError(RuntimeError):
    def __init__(self, name: str, status: int):
        msg = library().ozk_status_string(status).decode()
        super().__init__(f"{name} failed with status {status}: {msg}")
        self.status = status


def library() -> ctypes.CDLL:
    """The loaded libozk.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m fp64_gemm_emulation_ozk_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _call(name: str, *args) -> int:
    st = getattr(library(), name)(*args)
    if st != 0:
        raise OzkError(name, st)
    return st


def _stream(stream=None, *tensors):
    """The hipStream_t handle of `stream` (torch's current stream when None).  Tensors this
    binding allocated (outputs, workspace) come from torch's caching allocator on the
    current stream; when the work goes to another stream they are marked as used there,
    so that their memory is not handed out again before that stream's work ends."""
    if stream is None:
        stream = torch.cuda.current_stream()
    elif stream != torch.cuda.current_stream():
        for t in tensors:
            if t is not None:
                t.record_stream(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: torch.Tensor, dtype, name: str, ndim: int = 2):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA/HIP tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D")
    if ndim == 2 and t.numel() > 0 and t.stride(1) != 1:
        raise ValueError(f"{name} must be row-major with unit column stride")
    if ndim == 1 and t.numel() > 1 and t.stride(0) != 1:
        raise ValueError(f"{name} must be contiguous")


def _ld(t: torch.Tensor) -> int:
    return max(t.stride(0), t.shape[1], 1) if t.dim() == 2 else t.shape[-1]


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------- queries
def ozk_version() -> int:
    return library().ozk_version()


def ozk_moduli(r: int) -> list[int]:
    out = (ctypes.c_int32 * r)()
    _call("ozk_moduli", r, ctypes.cast(out, _ptr))
    return list(out)


def ozk_scaling_bits(r: int, k: int) -> tuple[int, int]:
    pa, pb = ctypes.c_int32(), ctypes.c_int32()
    _call("ozk_scaling_bits", r, k, ctypes.byref(pa), ctypes.byref(pb))
    return pa.value, pb.value


def ozk_scaling_bits_ex(r: int, k: int, scaling) -> tuple[int, int]:
    """(P_A, P_B) for the max rule, (alpha_A, alpha_B) for the norm rule."""
    pa, pb = ctypes.c_int32(), ctypes.c_int32()
    _call("ozk_scaling_bits_ex", r, k, _scaling(scaling), ctypes.byref(pa), ctypes.byref(pb))
    return pa.value, pb.value


def ozk_planes_ld(k: int) -> int:
    return library().ozk_planes_ld(k)


def _size_query(name: str, *args) -> int:
    out = ctypes.c_size_t()
    _call(name, *args, ctypes.byref(out))
    return out.value


def ozk_deconstruct_workspace_size(rows: int, cols: int, axis: int) -> int:
    return _size_query("ozk_deconstruct_workspace_size", rows, cols, axis)


def ozk_dgemm_workspace_size(m: int, n: int, k: int, r: int) -> int:
    return _size_query("ozk_dgemm_workspace_size", m, n, k, r)


def ozk_dgemv_workspace_size(m: int, k: int, nrhs: int, r: int, mode: int) -> int:
    return _size_query("ozk_dgemv_workspace_size", m, k, nrhs, r, mode)


def ozk_int8gemm_fp4limb_workspace_size(m: int, n: int, k: int) -> int:
    return _size_query("ozk_int8gemm_fp4limb_workspace_size", m, n, k)


# ----------------------------------------------------------------------------- operations
def _deconstruct(name: str, extra: tuple, x: torch.Tensor, axis: int, r: int,
                 k_budget, planes, exps, workspace, stream):
    _check(x, torch.float64, "x")
    rows, cols = x.shape
    kdim = cols if axis == 0 else rows
    lines = rows if axis == 0 else cols
    ldp = ozk_planes_ld(max(kdim, 1))
    if planes is None:
        planes = torch.empty((r, lines, ldp), dtype=torch.int8, device=x.device)
    if exps is None:
        exps = torch.empty(lines, dtype=torch.int32, device=x.device)
    ws_bytes = ozk_deconstruct_workspace_size(rows, cols, axis)
    if workspace is None and ws_bytes > 0:
        workspace = _workspace(ws_bytes, x.device)
    _call(name, _dev_ptr(x), rows, cols, _ld(x), axis, r,
          k_budget if k_budget is not None else kdim, *extra, _dev_ptr(planes),
          planes.shape[-1], planes.stride(0), _dev_ptr(exps), _dev_ptr(workspace),
          0 if workspace is None else workspace.numel(),
          _stream(stream, planes, exps, workspace))
    return planes, exps


def ozk_deconstruct(x: torch.Tensor, axis: int, r: int, k_budget: int | None = None,
                    planes: torch.Tensor | None = None, exps: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None, stream=None):
    """Residue planes [r][lines][ldp] (int8) and exponents [lines] (int32) of x."""
    return _deconstruct("ozk_deconstruct", (), x, axis, r, k_budget, planes, exps, workspace,
                        stream)


def ozk_deconstruct_ex(x: torch.Tensor, axis: int, r: int, scaling="max",
                       k_budget: int | None = None, planes: torch.Tensor | None = None,
                       exps: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                       stream=None):
    """ozk_deconstruct with a scaling rule ("max"/"norm" or OZK_SCALING_*)."""
    return _deconstruct("ozk_deconstruct_ex", (_scaling(scaling),), x, axis, r, k_budget,
                        planes, exps, workspace, stream)


def ozk_modular_products(planes_a: torch.Tensor, planes_b: torch.Tensor, r: int | None = None,
                         out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """int32 [r][m][n]: exact products of int8 planes [r][m][kp] and [r][n][kp]."""
    _check(planes_a, torch.int8, "planes_a", 3)
    _check(planes_b, torch.int8, "planes_b", 3)
    r = planes_a.shape[0] if r is None else r
    _, m, kp = planes_a.shape
    n = planes_b.shape[1]
    if out is None:
        out = torch.empty((r, m, n), dtype=torch.int32, device=planes_a.device)
    _call("ozk_modular_products", m, n, kp, r, _dev_ptr(planes_a), planes_a.stride(0),
          _dev_ptr(planes_b), planes_b.stride(0), _dev_ptr(out), out.stride(1), out.stride(0),
          _stream(stream, out))
    return out


def ozk_modular_residues(planes_a: torch.Tensor, planes_b: torch.Tensor, r: int | None = None,
                         out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """int8 [r][m][n]: symmetric residues of the exact plane products modulo m_l."""
    _check(planes_a, torch.int8, "planes_a", 3)
    _check(planes_b, torch.int8, "planes_b", 3)
    r = planes_a.shape[0] if r is None else r
    _, m, kp = planes_a.shape
    n = planes_b.shape[1]
    if out is None:
        out = torch.empty((r, m, n), dtype=torch.int8, device=planes_a.device)
    _call("ozk_modular_residues", m, n, kp, r, _dev_ptr(planes_a), planes_a.stride(0),
          _dev_ptr(planes_b), planes_b.stride(0), _dev_ptr(out), out.stride(1), out.stride(0),
          _stream(stream, out))
    return out


def ozk_reconstruct(products: torch.Tensor, exps_a: torch.Tensor, exps_b: torch.Tensor,
                    r: int | None = None, out: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """fp64 [m][n] from int32 products [r][m][n] and the exponents."""
    _check(products, torch.int32, "products", 3)
    _check(exps_a, torch.int32, "exps_a", 1)
    _check(exps_b, torch.int32, "exps_b", 1)
    r = products.shape[0] if r is None else r
    _, m, n = products.shape
    if out is None:
        out = torch.empty((m, n), dtype=torch.float64, device=products.device)
    _call("ozk_reconstruct", m, n, r, _dev_ptr(products), products.stride(1), products.stride(0),
          _dev_ptr(exps_a), _dev_ptr(exps_b), _dev_ptr(out), _ld(out), _stream(stream, out))
    return out


def _dgemm_args(a, b, r, out, workspace):
    _check(a, torch.float64, "A")
    _check(b, torch.float64, "B")
    m, k = a.shape
    kb, n = b.shape
    if kb != k:
        raise ValueError("inner dimensions differ")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float64, device=a.device)
    if workspace is None:
        workspace = _workspace(ozk_dgemm_workspace_size(m, n, k, r), a.device)
    return m, n, k, out, workspace


def ozk_dgemm(a: torch.Tensor, b: torch.Tensor, r: int, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Emulated fp64 C = A B through r moduli."""
    m, n, k, out, workspace = _dgemm_args(a, b, r, out, workspace)
    _call("ozk_dgemm", m, n, k, _dev_ptr(a), _ld(a), _dev_ptr(b), _ld(b), _dev_ptr(out), _ld(out),
          r, _dev_ptr(workspace), workspace.numel(), _stream(stream, out, workspace))
    return out


def ozk_dgemm_ex(a: torch.Tensor, b: torch.Tensor, r: int, scaling="max",
                 out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """ozk_dgemm with a scaling rule ("max"/"norm" or OZK_SCALING_*)."""
    m, n, k, out, workspace = _dgemm_args(a, b, r, out, workspace)
    _call("ozk_dgemm_ex", m, n, k, _dev_ptr(a), _ld(a), _dev_ptr(b), _ld(b), _dev_ptr(out),
          _ld(out), r, _scaling(scaling), _dev_ptr(workspace), workspace.numel(),
          _stream(stream, out, workspace))
    return out


def ozk_dgemm_ex_timed(a: torch.Tensor, b: torch.Tensor, r: int, gemm_start, gemm_stop,
                       scaling="max", out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """ozk_dgemm_ex that records two torch.cuda.Event objects (enable_timing=True, already
    recorded once so that they exist) around the launch of the residue products."""
    m, n, k, out, workspace = _dgemm_args(a, b, r, out, workspace)
    _call("ozk_dgemm_ex_timed", m, n, k, _dev_ptr(a), _ld(a), _dev_ptr(b), _ld(b),
          _dev_ptr(out), _ld(out), r, _scaling(scaling), _dev_ptr(workspace), workspace.numel(),
          _stream(stream, out, workspace), gemm_start.cuda_event, gemm_stop.cuda_event)
    return out


def ozk_dgemv(a: torch.Tensor | None, x: torch.Tensor, r: int, mode: int = 0,
              a_planes: torch.Tensor | None = None, a_exps: torch.Tensor | None = None,
              out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
              m: int | None = None, stream=None) -> torch.Tensor:
    """Emulated fp64 Y = A X for X with 1..32 columns (mode 0 on the fly, 1 stored)."""
    _check(x, torch.float64, "X")
    k, nrhs = x.shape
    if a is not None:
        _check(a, torch.float64, "A")
        m = a.shape[0]
    elif a_planes is not None:
        m = a_planes.shape[1]
    if m is None:
        raise ValueError("m unknown")
    if out is None:
        out = torch.empty((m, nrhs), dtype=torch.float64, device=x.device)
    if workspace is None:
        workspace = _workspace(ozk_dgemv_workspace_size(m, k, nrhs, r, mode), x.device)
    ldp = a_planes.shape[-1] if a_planes is not None else 0
    pstride = a_planes.stride(0) if a_planes is not None else 0
    _call("ozk_dgemv", m, k, nrhs, _dev_ptr(a), _ld(a) if a is not None else k,
          _dev_ptr(a_planes), ldp, pstride, _dev_ptr(a_exps), _dev_ptr(x), _ld(x),
          _dev_ptr(out), _ld(out), r, mode, _dev_ptr(workspace), workspace.numel(),
          _stream(stream, out, workspace))
    return out


def ozk_dgemv_noalloc(a: torch.Tensor | None, x: torch.Tensor, r: int, mode: int = 0,
                      a_planes: torch.Tensor | None = None, a_exps: torch.Tensor | None = None,
                      out: torch.Tensor | None = None, m: int | None = None,
                      stream=None) -> torch.Tensor:
    """ozk_dgemv through the allocation-free entry point: the library's fixed scratch
    array (OZK_NOALLOC_SCRATCH_BYTES per GPU) instead of a workspace.  With `out` given
    nothing is allocated at all; calls that overlap in time on one GPU race."""
    _check(x, torch.float64, "X")
    k, nrhs = x.shape
    if a is not None:
        _check(a, torch.float64, "A")
        m = a.shape[0]
    elif a_planes is not None:
        m = a_planes.shape[1]
    if m is None:
        raise ValueError("m unknown")
    if out is None:
        out = torch.empty((m, nrhs), dtype=torch.float64, device=x.device)
    ldp = a_planes.shape[-1] if a_planes is not None else 0
    pstride = a_planes.stride(0) if a_planes is not None else 0
    _call("ozk_dgemv_noalloc", m, k, nrhs, _dev_ptr(a), _ld(a) if a is not None else k,
          _dev_ptr(a_planes), ldp, pstride, _dev_ptr(a_exps), _dev_ptr(x), _ld(x),
          _dev_ptr(out), _ld(out), r, mode, _stream(stream, out))
    return out


def ozk_spmv_csr_workspace_size(rows: int, cols: int, r: int) -> int:
    return _size_query("ozk_spmv_csr_workspace_size", rows, cols, r)


def ozk_spmv_csr(row_ptr: torch.Tensor, col_idx: torch.Tensor, vals: torch.Tensor,
                 x: torch.Tensor, r: int, max_row_nnz: int | None = None,
                 out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """Emulated fp64 y = A x for A in CSR (int32 row_ptr / col_idx, float64 vals).
    max_row_nnz bounds the entries of a row (it sets the bit budget); when omitted it
    is read from row_ptr, which synchronises with the device."""
    _check(row_ptr, torch.int32, "row_ptr", 1)
    _check(col_idx, torch.int32, "col_idx", 1)
    _check(vals, torch.float64, "vals", 1)
    _check(x, torch.float64, "x", 1)
    rows, cols, nnz = row_ptr.shape[0] - 1, x.shape[0], vals.shape[0]
    if col_idx.shape[0] != nnz:
        raise ValueError("col_idx and vals differ in length")
    if max_row_nnz is None:
        max_row_nnz = max(int(torch.diff(row_ptr).max().item()) if rows > 0 else 1, 1)
    if out is None:
        out = torch.empty(rows, dtype=torch.float64, device=x.device)
    if workspace is None:
        workspace = _workspace(ozk_spmv_csr_workspace_size(rows, cols, r), x.device)
    _call("ozk_spmv_csr", rows, cols, nnz, _dev_ptr(row_ptr), _dev_ptr(col_idx), _dev_ptr(vals),
          max_row_nnz, _dev_ptr(x), _dev_ptr(out), r, _dev_ptr(workspace), workspace.numel(),
          _stream(stream, out, workspace))
    return out


def ozk_fp4limb_pack(x: torch.Tensor, axis: int, planes: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    """Packed e2m1 digit planes uint8 [3][lines][ldp_bytes] of an int8 matrix."""
    _check(x, torch.int8, "x")
    rows, cols = x.shape
    kdim = cols if axis == 0 else rows
    lines = rows if axis == 0 else cols
    ldpb = ozk_planes_ld(max(kdim, 1)) // 2
    if planes is None:
        planes = torch.empty((3, lines, ldpb), dtype=torch.uint8, device=x.device)
    _call("ozk_fp4limb_pack", _dev_ptr(x), rows, cols, _ld(x), axis, _dev_ptr(planes),
          planes.shape[-1], planes.stride(0), _stream(stream, planes))
    return planes


def ozk_fp4limb_products(planes_a: torch.Tensor, planes_b: torch.Tensor,
                         out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The 9 exact digit products int32 [9][m][n] (index 3*da + db)."""
    _check(planes_a, torch.uint8, "planes_a", 3)
    _check(planes_b, torch.uint8, "planes_b", 3)
    _, m, ldpb = planes_a.shape
    n = planes_b.shape[1]
    if out is None:
        out = torch.empty((9, m, n), dtype=torch.int32, device=planes_a.device)
    _call("ozk_fp4limb_products", m, n, ldpb, _dev_ptr(planes_a), planes_a.stride(0),
          _dev_ptr(planes_b), planes_b.stride(0), _dev_ptr(out), out.stride(1), out.stride(0),
          _stream(stream, out))
    return out


def ozk_int8gemm_fp4limb(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Exact int32 C = A B for int8 A, B through 9 FP4 limb GEMMs."""
    _check(a, torch.int8, "A")
    _check(b, torch.int8, "B")
    m, k = a.shape
    n = b.shape[1]
    if out is None:
        out = torch.empty((m, n), dtype=torch.int32, device=a.device)
    if workspace is None:
        workspace = _workspace(ozk_int8gemm_fp4limb_workspace_size(m, n, k), a.device)
    _call("ozk_int8gemm_fp4limb", m, n, k, _dev_ptr(a), _ld(a), _dev_ptr(b), _ld(b),
          _dev_ptr(out), _ld(out), _dev_ptr(workspace), workspace.numel(),
          _stream(stream, out, workspace))
    return out


# ------------------------------------------------------------ 6-product FP4 INT8 GEMM
def ozk_fp4awe_line_bytes(k: int) -> int:
    return library().ozk_fp4awe_line_bytes(k)


def ozk_int8gemm_fp4awe_workspace_size(m: int, n: int, k: int) -> int:
    return _size_query("ozk_int8gemm_fp4awe_workspace_size", m, n, k)


def ozk_fp4awe_pack(x: torch.Tensor, axis: int, planes: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """Packed 6-product planes uint8 [lines][line_bytes] of an int8 matrix (axis 0: rows
    are lines, K = columns; axis 1: columns are lines, K = rows)."""
    _check(x, torch.int8, "x")
    rows, cols = x.shape
    kdim = cols if axis == 0 else rows
    lines = rows if axis == 0 else cols
    if planes is None:
        planes = torch.empty((lines, ozk_fp4awe_line_bytes(max(kdim, 1))), dtype=torch.uint8,
                             device=x.device)
    _call("ozk_fp4awe_pack", _dev_ptr(x), rows, cols, _ld(x), axis, _dev_ptr(planes),
          planes.stride(0), _stream(stream, planes))
    return planes


def ozk_fp4awe_products(planes_a: torch.Tensor, planes_b: torch.Tensor, k: int,
                        out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The 6 exact plane products int32 [6][m][n] from packed lines of A and B."""
    _check(planes_a, torch.uint8, "planes_a")
    _check(planes_b, torch.uint8, "planes_b")
    m, n = planes_a.shape[0], planes_b.shape[0]
    if out is None:
        out = torch.empty((6, m, n), dtype=torch.int32, device=planes_a.device)
    _call("ozk_fp4awe_products", m, n, k, _dev_ptr(planes_a), planes_a.stride(0),
          _dev_ptr(planes_b), planes_b.stride(0), _dev_ptr(out), out.stride(1), out.stride(0),
          _stream(stream, out))
    return out


def ozk_int8gemm_fp4awe(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Exact int32 C = A B for int8 A, B through 6 FP4 plane products."""
    _check(a, torch.int8, "A")
    _check(b, torch.int8, "B")
    m, k = a.shape
    n = b.shape[1]
    if out is None:
        out = torch.empty((m, n), dtype=torch.int32, device=a.device)
    if workspace is None:
        workspace = _workspace(ozk_int8gemm_fp4awe_workspace_size(m, n, k), a.device)
    _call("ozk_int8gemm_fp4awe", m, n, k, _dev_ptr(a), _ld(a), _dev_ptr(b), _ld(b),
          _dev_ptr(out), _ld(out), _dev_ptr(workspace), workspace.numel(),
          _stream(stream, out, workspace))
    return out


# ------------------------------------------------------------ 4-product FP4 INT4 x INT8 GEMM
def ozk_fp4awe4_line_bytes(k: int) -> int:
    return library().ozk_fp4awe4_line_bytes(k)


def ozk_int4int8gemm_fp4awe_workspace_size(m: int, n: int, k: int) -> int:
    return _size_query("ozk_int4int8gemm_fp4awe_workspace_size", m, n, k)


def ozk_fp4awe4_pack(x: torch.Tensor, axis: int, int4: bool,
                     planes: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Packed 4-product planes uint8 [lines][line_bytes] of an int4 (low nibbles, int4=True)
    or int8 matrix (axis 0: rows are lines, K = columns; axis 1: columns are lines)."""
    _check(x, torch.int8, "x")
    rows, cols = x.shape
    kdim = cols if axis == 0 else rows
    lines = rows if axis == 0 else cols
    if planes is None:
        planes = torch.empty((lines, ozk_fp4awe4_line_bytes(max(kdim, 1))), dtype=torch.uint8,
                             device=x.device)
    _call("ozk_fp4awe4_pack", _dev_ptr(x), rows, cols, _ld(x), axis, 1 if int4 else 0,
          _dev_ptr(planes), planes.stride(0), _stream(stream, planes))
    return planes


def ozk_fp4awe4_products(planes_a: torch.Tensor, planes_b: torch.Tensor, k: int,
                         out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The 4 exact plane products int32 [4][m][n] from packed lines of A and B."""
    _check(planes_a, torch.uint8, "planes_a")
    _check(planes_b, torch.uint8, "planes_b")
    m, n = planes_a.shape[0], planes_b.shape[0]
    if out is None:
        out = torch.empty((4, m, n), dtype=torch.int32, device=planes_a.device)
    _call("ozk_fp4awe4_products", m, n, k, _dev_ptr(planes_a), planes_a.stride(0),
          _dev_ptr(planes_b), planes_b.stride(0), _dev_ptr(out), out.stride(1), out.stride(0),
          _stream(stream, out))
    return out


def ozk_int4int8gemm_fp4awe(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Exact int32 C = A B for an int4 A (one value per byte, low nibble) and an int8 B
    through 4 FP4 plane products."""
    _check(a, torch.int8, "A")
    _check(b, torch.int8, "B")
    m, k = a.shape
    n = b.shape[1]
    if out is None:
        out = torch.empty((m, n), dtype=torch.int32, device=a.device)
    if workspace is None:
        workspace = _workspace(ozk_int4int8gemm_fp4awe_workspace_size(m, n, k), a.device)
    _call("ozk_int4int8gemm_fp4awe", m, n, k, _dev_ptr(a), _ld(a), _dev_ptr(b), _ld(b),
          _dev_ptr(out), _ld(out), _dev_ptr(workspace), workspace.numel(),
          _stream(stream, out, workspace))
    return out
