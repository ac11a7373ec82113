// extern "C" entry points of libozk.so: argument validation (before any HIP call),
// workspace carving, and the stream-ordered launch sequence of each operation.
#include <hip/hip_runtime.h>

#include "ozk_internal.h"

using namespace ozk;

namespace {

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Workspace carving: consecutive 256-byte aligned regions.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  }
};

// Scratch of one operand's deconstruction beyond its planes and exponents: the line
// maxima of the max rule, or the chunk partials of the norm rule; the larger of the two,
// so that one workspace query serves both rules.  None for rows the fused kernel takes.
size_t deconstruct_scratch(int64_t rows, int64_t cols, int axis) {
  if (axis == 0 && rows_fused_supported(cols)) return 0;
  const int64_t lines = axis == 0 ? rows : cols;
  const size_t maxb = align256((size_t)lines * 8);
  const size_t part = 2 * align256((size_t)lines * norm_chunks(rows, cols, axis) * 8);
  return maxb > part ? maxb : part;
}

struct DgemmLayout {
  int64_t kp;
  size_t planes_a, planes_b, residues, exps_a, exps_b, scr_a, scr_b;
  size_t total() const {
    return align256(planes_a) + align256(planes_b) + align256(residues) + align256(exps_a) +
           align256(exps_b) + align256(scr_a) + align256(scr_b);
  }
};

DgemmLayout dgemm_layout(int64_t m, int64_t n, int64_t k, int r) {
  DgemmLayout L;
  // K padded to whole 128-byte rows: the products then stream whole cache lines.
  L.kp = round_up(k, 2 * kPlaneK);
  L.planes_a = (size_t)r * m * L.kp;
  L.planes_b = (size_t)r * n * L.kp;
  L.residues = (size_t)r * m * n;
  L.exps_a = (size_t)m * 4;
  L.exps_b = (size_t)n * 4;
  L.scr_a = deconstruct_scratch(m, k, 0);
  L.scr_b = deconstruct_scratch(k, n, 1);
  return L;
}

int check_r(int r) { return (r >= 1 && r <= kMaxModuli) ? OZK_OK : OZK_EINVAL; }

// First pass of a column deconstruction: the column maxima (max rule, into scratch as
// maxbits) or the norm-rule exponents (chunk partials in scratch, exponents into exps).
int cols_prep(const double* x, int64_t rows, int64_t cols, int64_t ldx, int scaling, int width,
              void* scratch, int32_t* exps, hipStream_t s) {
  int st;
  if (scaling == OZK_SCALING_NORM) {
    Carver cv(scratch);
    const size_t n = (size_t)cols * norm_chunks(rows, cols, 1) * 8;
    uint64_t* pmax = static_cast<uint64_t*>(cv.take(n));
    double* ps = static_cast<double*>(cv.take(n));
    return launch_norm_exps(x, rows, cols, ldx, 1, width, pmax, ps, exps, s);
  }
  uint64_t* maxbits = static_cast<uint64_t*>(scratch);
  if ((st = launch_fill_u64(maxbits, cols, 0, s)) != OZK_OK) return st;
  return launch_absmax(x, rows, cols, ldx, 1, maxbits, s);
}

// Deconstruct one operand (axis 0: per-row, axis 1: per-column) into planes by either
// scaling rule; width is P (max rule) or alpha (norm rule) of this operand and scratch
// holds deconstruct_scratch(rows, cols, axis) bytes.
int deconstruct_impl(const double* x, int64_t rows, int64_t cols, int64_t ldx, int axis, int r,
                     int scaling, int width, int8_t* planes, int64_t ldp, int64_t plane_stride,
                     int32_t* exps, void* scratch, hipStream_t s) {
  int st;
  if (axis == 0 && rows_fused_supported(cols))
    return launch_residues_rows_fused(x, rows, cols, ldx, r, scaling, width, planes, ldp,
                                      plane_stride, exps, s);
  const int norm = scaling == OZK_SCALING_NORM;
  if (axis == 1) {
    if ((st = cols_prep(x, rows, cols, ldx, scaling, width, scratch, exps, s)) != OZK_OK)
      return st;
    return launch_residues(x, rows, cols, ldx, 1, r, width,
                           static_cast<const uint64_t*>(scratch), planes, ldp, plane_stride,
                           exps, norm, s);
  }
  if (norm) {
    Carver cv(scratch);
    const size_t n = (size_t)rows * norm_chunks(rows, cols, 0) * 8;
    uint64_t* pmax = static_cast<uint64_t*>(cv.take(n));
    double* ps = static_cast<double*>(cv.take(n));
    if ((st = launch_norm_exps(x, rows, cols, ldx, 0, width, pmax, ps, exps, s)) != OZK_OK)
      return st;
    return launch_residues(x, rows, cols, ldx, 0, r, width, nullptr, planes, ldp,
                           plane_stride, exps, 1, s);
  }
  uint64_t* maxbits = static_cast<uint64_t*>(scratch);
  if ((st = launch_fill_u64(maxbits, rows, 0, s)) != OZK_OK) return st;
  if ((st = launch_absmax(x, rows, cols, ldx, 0, maxbits, s)) != OZK_OK) return st;
  return launch_residues(x, rows, cols, ldx, 0, r, width, maxbits, planes, ldp, plane_stride,
                         exps, 0, s);
}

// Both operands of a product: B's first pass, then A's rows and B's residues in one
// launch where that applies, else one operand after the other.
int deconstruct_operands(const double* A, int64_t m, int64_t k, int64_t lda, const double* B,
                         int64_t n, int64_t ldb, int r, int scaling, int wa, int wb,
                         int8_t* planes_a, int8_t* planes_b, int64_t kp, int32_t* exps_a,
                         int32_t* exps_b, void* scr_a, void* scr_b, hipStream_t s) {
  int st;
  if (!rows_fused_supported(k) || k > 8192) {
    if ((st = deconstruct_impl(A, m, k, lda, 0, r, scaling, wa, planes_a, kp, m * kp, exps_a,
                               scr_a, s)))
      return st;
    return deconstruct_impl(B, k, n, ldb, 1, r, scaling, wb, planes_b, kp, n * kp, exps_b,
                            scr_b, s);
  }
  if ((st = cols_prep(B, k, n, ldb, scaling, wb, scr_b, exps_b, s)) != OZK_OK) return st;
  st = launch_deconstruct_pair(A, m, k, lda, B, n, ldb, r, scaling, wa, wb,
                               static_cast<const uint64_t*>(scr_b), planes_a, planes_b, kp,
                               exps_a, exps_b, s);
  if (st != OZK_EUNSUPPORTED) return st;
  if ((st = launch_residues_rows_fused(A, m, k, lda, r, scaling, wa, planes_a, kp, m * kp,
                                       exps_a, s)))
    return st;
  return launch_residues(B, k, n, ldb, 1, r, wb, static_cast<const uint64_t*>(scr_b), planes_b,
                         kp, n * kp, exps_b, scaling == OZK_SCALING_NORM, s);
}

}  // namespace

extern "C" {

int ozk_version(void) { return 100; }

const char* ozk_status_string(int status) {
  switch (status) {
    case OZK_OK: return "success";
    case OZK_EINVAL: return "invalid argument";
    case OZK_EWORKSPACE: return "workspace missing or too small";
    case OZK_ERANGE: return "inner dimension out of range for exact products or the bit budget";
    case OZK_EHIP: return "HIP launch failed";
    case OZK_EUNSUPPORTED: return "unsupported request";
    case OZK_ENOSCRATCH:
      return "request needs more scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

int ozk_moduli(int r, int32_t* out) { return moduli_list(r, out); }

int ozk_scaling_bits(int r, int64_t k, int32_t* pa, int32_t* pb) {
  int a = 0, b = 0;
  int st = scaling_bits(r, k, &a, &b);
  if (st != OZK_OK) return st;
  if (pa) *pa = a;
  if (pb) *pb = b;
  return OZK_OK;
}

int ozk_scaling_bits_ex(int r, int64_t k, int scaling, int32_t* pa, int32_t* pb) {
  int a = 0, b = 0;
  int st = scaling_widths(scaling, r, k, &a, &b);
  if (st != OZK_OK) return st;
  if (pa) *pa = a;
  if (pb) *pb = b;
  return OZK_OK;
}

int64_t ozk_planes_ld(int64_t k) { return k <= 0 ? 0 : round_up(k, kPlaneK); }

int ozk_deconstruct_workspace_size(int64_t rows, int64_t cols, int axis, size_t* bytes) {
  if (!bytes || rows < 0 || cols < 0 || (axis != 0 && axis != 1)) return OZK_EINVAL;
  *bytes = deconstruct_scratch(rows, cols, axis);
  return OZK_OK;
}

int ozk_deconstruct_ex(const double* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                       int r, int64_t k_budget, int scaling, int8_t* planes, int64_t ldp,
                       int64_t plane_stride, int32_t* exps, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (axis != 0 && axis != 1) return OZK_EINVAL;
  if (scaling != OZK_SCALING_MAX && scaling != OZK_SCALING_NORM) return OZK_EINVAL;
  if (check_r(r) != OZK_OK) return OZK_EINVAL;
  if (rows < 0 || cols < 0 || ldx < (cols > 0 ? cols : 1)) return OZK_EINVAL;
  const int64_t K = axis == 0 ? cols : rows;
  const int64_t lines = axis == 0 ? rows : cols;
  if (ldp < K || ldp % kPlaneK != 0 || ldp <= 0) return OZK_EINVAL;
  if (plane_stride < lines * ldp || plane_stride % kPlaneK != 0) return OZK_EINVAL;
  int wa = 0, wb = 0;
  int st = scaling_widths(scaling, r, k_budget, &wa, &wb);
  if (st != OZK_OK) return st;
  if (lines == 0) return OZK_OK;
  if (!planes || !exps || (K > 0 && !x)) return OZK_EINVAL;
  if (!aligned(planes, 16)) return OZK_EINVAL;
  const size_t need = deconstruct_scratch(rows, cols, axis);
  if (need > workspace_bytes || (need > 0 && !workspace)) return OZK_EWORKSPACE;
  if (need > 0 && !aligned(workspace, 8)) return OZK_EINVAL;
  return deconstruct_impl(x, rows, cols, ldx, axis, r, scaling, axis == 0 ? wa : wb, planes,
                          ldp, plane_stride, exps, workspace, as_stream(stream));
}

int ozk_deconstruct(const double* x, int64_t rows, int64_t cols, int64_t ldx, int axis, int r,
                    int64_t k_budget, int8_t* planes, int64_t ldp, int64_t plane_stride,
                    int32_t* exps, void* workspace, size_t workspace_bytes, void* stream) {
  return ozk_deconstruct_ex(x, rows, cols, ldx, axis, r, k_budget, OZK_SCALING_MAX, planes, ldp,
                            plane_stride, exps, workspace, workspace_bytes, stream);
}

int ozk_modular_products(int64_t m, int64_t n, int64_t kp, int r, const int8_t* pa,
                         int64_t stride_a, const int8_t* pb, int64_t stride_b,
                         int32_t* products, int64_t ldp_out, int64_t stride_p, void* stream) {
  if (check_r(r) != OZK_OK) return OZK_EINVAL;
  if (m < 0 || n < 0 || kp <= 0 || kp % kPlaneK != 0) return OZK_EINVAL;
  if (kp > round_up(OZK_MAX_K, kPlaneK)) return OZK_ERANGE;
  if (ldp_out < (n > 0 ? n : 1) || stride_p < m * ldp_out) return OZK_EINVAL;
  if (stride_a < m * kp || stride_b < n * kp) return OZK_EINVAL;
  if (stride_a % 16 || stride_b % 16) return OZK_EINVAL;
  if (m == 0 || n == 0) return OZK_OK;
  if (!pa || !pb || !products || !aligned(pa, 16) || !aligned(pb, 16)) return OZK_EINVAL;
  return launch_gemm_i8(m, n, kp, r, pa, stride_a, pb, stride_b, products, ldp_out, stride_p,
                        kEpiProducts, as_stream(stream));
}

int ozk_modular_residues(int64_t m, int64_t n, int64_t kp, int r, const int8_t* pa,
                         int64_t stride_a, const int8_t* pb, int64_t stride_b, int8_t* residues,
                         int64_t ldr, int64_t stride_r, void* stream) {
  if (check_r(r) != OZK_OK) return OZK_EINVAL;
  if (m < 0 || n < 0 || kp <= 0 || kp % kPlaneK != 0) return OZK_EINVAL;
  if (kp > round_up(OZK_MAX_K, kPlaneK)) return OZK_ERANGE;
  if (ldr < (n > 0 ? n : 1) || stride_r < m * ldr) return OZK_EINVAL;
  if (stride_a < m * kp || stride_b < n * kp) return OZK_EINVAL;
  if (stride_a % 16 || stride_b % 16) return OZK_EINVAL;
  if (m == 0 || n == 0) return OZK_OK;
  if (!pa || !pb || !residues || !aligned(pa, 16) || !aligned(pb, 16)) return OZK_EINVAL;
  return launch_gemm_i8(m, n, kp, r, pa, stride_a, pb, stride_b, residues, ldr, stride_r,
                        kEpiResidues, as_stream(stream));
}

int ozk_reconstruct(int64_t m, int64_t n, int r, const int32_t* products, int64_t ldp_in,
                    int64_t stride_p, const int32_t* exps_a, const int32_t* exps_b, double* C,
                    int64_t ldc, void* stream) {
  if (check_r(r) != OZK_OK) return OZK_EINVAL;
  if (m < 0 || n < 0) return OZK_EINVAL;
  if (ldp_in < (n > 0 ? n : 1) || stride_p < m * ldp_in || ldc < (n > 0 ? n : 1))
    return OZK_EINVAL;
  if (m == 0 || n == 0) return OZK_OK;
  if (!products || !exps_a || !exps_b || !C) return OZK_EINVAL;
  return launch_crt(m, n, r, products, 1, ldp_in, stride_p, exps_a, exps_b, C, ldc,
                    as_stream(stream));
}

int ozk_dgemm_workspace_size(int64_t m, int64_t n, int64_t k, int r, size_t* bytes) {
  if (!bytes || m < 0 || n < 0 || k < 1 || check_r(r) != OZK_OK) return OZK_EINVAL;
  if (k > OZK_MAX_K) return OZK_ERANGE;
  *bytes = dgemm_layout(m, n, k, r).total();
  return OZK_OK;
}

int ozk_dgemm_ex(int64_t m, int64_t n, int64_t k, const double* A, int64_t lda,
                 const double* B, int64_t ldb, double* C, int64_t ldc, int r, int scaling,
                 void* workspace, size_t workspace_bytes, void* stream) {
  return ozk_dgemm_ex_timed(m, n, k, A, lda, B, ldb, C, ldc, r, scaling, workspace,
                            workspace_bytes, stream, nullptr, nullptr);
}

int ozk_dgemm_ex_timed(int64_t m, int64_t n, int64_t k, const double* A, int64_t lda,
                       const double* B, int64_t ldb, double* C, int64_t ldc, int r, int scaling,
                       void* workspace, size_t workspace_bytes, void* stream,
                       void* gemm_start, void* gemm_stop) {
  if ((gemm_start == nullptr) != (gemm_stop == nullptr)) return OZK_EINVAL;
  if (check_r(r) != OZK_OK) return OZK_EINVAL;
  if (scaling != OZK_SCALING_MAX && scaling != OZK_SCALING_NORM) return OZK_EINVAL;
  if (m < 0 || n < 0 || k < 1) return OZK_EINVAL;
  if (k > OZK_MAX_K) return OZK_ERANGE;
  if (lda < k || ldb < (n > 0 ? n : 1) || ldc < (n > 0 ? n : 1)) return OZK_EINVAL;
  int wa = 0, wb = 0;
  int st = scaling_widths(scaling, r, k, &wa, &wb);
  if (st != OZK_OK) return st;
  if (m == 0 || n == 0) return OZK_OK;
  if (!A || !B || !C) return OZK_EINVAL;
  const DgemmLayout L = dgemm_layout(m, n, k, r);
  if (!workspace || workspace_bytes < L.total()) return OZK_EWORKSPACE;
  if (!aligned(workspace, 256)) return OZK_EINVAL;
  if ((size_t)m * n > (size_t)0x7fffffffffffull) return OZK_EUNSUPPORTED;
  Carver cv(workspace);
  int8_t* planes_a = static_cast<int8_t*>(cv.take(L.planes_a));
  int8_t* planes_b = static_cast<int8_t*>(cv.take(L.planes_b));
  int8_t* residues = static_cast<int8_t*>(cv.take(L.residues));
  int32_t* exps_a = static_cast<int32_t*>(cv.take(L.exps_a));
  int32_t* exps_b = static_cast<int32_t*>(cv.take(L.exps_b));
  void* scr_a = cv.take(L.scr_a);
  void* scr_b = cv.take(L.scr_b);
  hipStream_t s = as_stream(stream);
  const int64_t kp = L.kp;
  if ((st = deconstruct_operands(A, m, k, lda, B, n, ldb, r, scaling, wa, wb, planes_a,
                                 planes_b, kp, exps_a, exps_b, scr_a, scr_b, s)))
    return st;
  if ((st = launch_gemm_i8(m, n, kp, r, planes_a, m * kp, planes_b, n * kp, residues, n, m * n,
                           kEpiResidues, s, static_cast<hipEvent_t>(gemm_start),
                           static_cast<hipEvent_t>(gemm_stop))))
    return st;
  return launch_crt(m, n, r, residues, 0, n, m * n, exps_a, exps_b, C, ldc, s);
}

int ozk_dgemm(int64_t m, int64_t n, int64_t k, const double* A, int64_t lda, const double* B,
              int64_t ldb, double* C, int64_t ldc, int r, void* workspace,
              size_t workspace_bytes, void* stream) {
  return ozk_dgemm_ex(m, n, k, A, lda, B, ldb, C, ldc, r, OZK_SCALING_MAX, workspace,
                      workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- emulated DGEMV
namespace {

struct GemvLayout {
  int64_t kp;
  bool digits;   // on the fly through base-256 digits (scaling bits of A <= 50)
  size_t x_planes, x_exps, x_max, res, a_exps, a_max, xd, corr, part;
  size_t total() const {
    return align256(x_planes) + align256(x_exps) + align256(x_max) + align256(res) +
           align256(a_exps) + align256(a_max) + align256(xd) + align256(corr) +
           align256(part);
  }
};

GemvLayout gemv_layout(int64_t m, int64_t k, int64_t nrhs, int r, int mode) {
  GemvLayout L;
  L.kp = round_up(k, kPlaneK);
  L.x_planes = (size_t)r * nrhs * L.kp;
  L.x_exps = (size_t)nrhs * 4;
  L.x_max = (size_t)nrhs * 8;
  L.res = (size_t)r * m * nrhs;
  L.a_exps = mode == 0 ? (size_t)m * 4 : 0;
  L.a_max = mode == 0 ? (size_t)m * 8 : 0;
  int pa = 0, pb = 0;
  L.digits = mode == 0 && scaling_bits(r, k, &pa, &pb) == OZK_OK &&
             gemv_digits_supported(pa, (int64_t)r * nrhs);
  L.xd = L.corr = L.part = 0;
  if (L.digits) gemv_digits_workspace(m, L.kp, r, nrhs, &L.xd, &L.corr, &L.part);
  return L;
}

}  // namespace

extern "C" {

int ozk_dgemv_workspace_size(int64_t m, int64_t k, int64_t nrhs, int r, int mode,
                             size_t* bytes) {
  if (!bytes || m < 0 || k < 1 || nrhs < 1 || nrhs > 32 || check_r(r) != OZK_OK) return OZK_EINVAL;
  if (mode != 0 && mode != 1) return OZK_EINVAL;
  if (k > OZK_MAX_K) return OZK_ERANGE;
  *bytes = gemv_layout(m, k, nrhs, r, mode).total();
  return OZK_OK;
}

}  // extern "C"

namespace ozk {

int dgemv_validate(int64_t m, int64_t k, int64_t nrhs, const double* A, int64_t lda,
                   const int8_t* A_planes, int64_t ldp, int64_t plane_stride,
                   const int32_t* A_exps, const double* X, int64_t ldx, const double* Y,
                   int64_t ldy, int r, int mode) {
  if (check_r(r) != OZK_OK || (mode != 0 && mode != 1)) return OZK_EINVAL;
  if (m < 0 || k < 1 || nrhs < 1 || nrhs > 32) return OZK_EINVAL;
  if (k > OZK_MAX_K) return OZK_ERANGE;
  if (ldx < nrhs || ldy < nrhs) return OZK_EINVAL;
  int pa = 0, pb = 0;
  int st = scaling_bits(r, k, &pa, &pb);
  if (st != OZK_OK) return st;
  const int64_t kp = round_up(k, kPlaneK);
  if (mode == 0) {
    if (lda < k) return OZK_EINVAL;
  } else {
    if (ldp < kp || ldp % kPlaneK != 0 || plane_stride < m * ldp || plane_stride % 16 != 0)
      return OZK_EINVAL;
  }
  if (m == 0) return OZK_OK;
  if (!X || !Y) return OZK_EINVAL;
  if (mode == 0 && !A) return OZK_EINVAL;
  if (mode == 1 && (!A_planes || !A_exps || !aligned(A_planes, 16))) return OZK_EINVAL;
  return OZK_OK;
}

}  // namespace ozk

extern "C" {

int ozk_dgemv(int64_t m, int64_t k, int64_t nrhs, const double* A, int64_t lda,
              const int8_t* A_planes, int64_t ldp, int64_t plane_stride, const int32_t* A_exps,
              const double* X, int64_t ldx, double* Y, int64_t ldy, int r, int mode,
              void* workspace, size_t workspace_bytes, void* stream) {
  int st = dgemv_validate(m, k, nrhs, A, lda, A_planes, ldp, plane_stride, A_exps, X, ldx, Y,
                          ldy, r, mode);
  if (st != OZK_OK || m == 0) return st;
  int pa = 0, pb = 0;
  scaling_bits(r, k, &pa, &pb);
  const GemvLayout L = gemv_layout(m, k, nrhs, r, mode);
  if (!workspace || workspace_bytes < L.total()) return OZK_EWORKSPACE;
  if (!aligned(workspace, 256)) return OZK_EINVAL;
  Carver cv(workspace);
  int8_t* x_planes = static_cast<int8_t*>(cv.take(L.x_planes));
  int32_t* x_exps = static_cast<int32_t*>(cv.take(L.x_exps));
  uint64_t* x_max = static_cast<uint64_t*>(cv.take(L.x_max));
  int8_t* res = static_cast<int8_t*>(cv.take(L.res));
  int32_t* a_exps = static_cast<int32_t*>(cv.take(L.a_exps));
  uint64_t* a_max = static_cast<uint64_t*>(cv.take(L.a_max));
  int8_t* xd = static_cast<int8_t*>(cv.take(L.xd));
  int32_t* corr = static_cast<int32_t*>(cv.take(L.corr));
  int8_t* part = static_cast<int8_t*>(cv.take(L.part));
  hipStream_t s = as_stream(stream);
  const int64_t kp = L.kp;
  if ((st = deconstruct_impl(X, k, nrhs, ldx, 1, r, OZK_SCALING_MAX, pb, x_planes, kp, nrhs * kp,
                             x_exps, x_max, s)))
    return st;
  const int32_t* ea = A_exps;
  if (mode == 0) {
    if (!ea) {
      if ((st = launch_line_exps(A, m, k, lda, 0, pa, a_max, a_exps, s))) return st;
      ea = a_exps;
    }
    if (L.digits)
      st = launch_gemv_digits(A, m, k, lda, ea, r, x_planes, kp, nrhs * kp, (int)nrhs, xd, corr,
                              part, res, s);
    else
      st = launch_gemv_fly(A, m, k, lda, ea, r, pa, x_planes, kp, nrhs * kp, (int)nrhs, res, s);
  } else {
    st = launch_gemv_stored(m, kp, r, A_planes, ldp, plane_stride, x_planes, nrhs * kp,
                            (int)nrhs, res, s);
  }
  if (st) return st;
  return launch_crt(m, nrhs, r, res, 0, nrhs, m * nrhs, ea, x_exps, Y, ldy, s);
}

// ---------------------------------------------------------------- FP4-limb INT8 GEMM
int ozk_fp4limb_pack(const int8_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                     uint8_t* planes, int64_t ldp_bytes, int64_t plane_stride, void* stream) {
  if (axis != 0 && axis != 1) return OZK_EINVAL;
  if (rows < 0 || cols < 0 || ldx < (cols > 0 ? cols : 1)) return OZK_EINVAL;
  const int64_t K = axis == 0 ? cols : rows;
  const int64_t lines = axis == 0 ? rows : cols;
  if (ldp_bytes <= 0 || ldp_bytes % 32 != 0 || 2 * ldp_bytes < K) return OZK_EINVAL;
  if (plane_stride < lines * ldp_bytes || plane_stride % 16 != 0) return OZK_EINVAL;
  if (lines == 0) return OZK_OK;
  if (!planes || (K > 0 && !x) || !aligned(planes, 16)) return OZK_EINVAL;
  return launch_fp4_pack(x, rows, cols, ldx, axis, planes, ldp_bytes, plane_stride,
                         as_stream(stream));
}

int ozk_fp4limb_products(int64_t m, int64_t n, int64_t ldp_bytes, const uint8_t* planes_a,
                         int64_t stride_a, const uint8_t* planes_b, int64_t stride_b,
                         int32_t* products, int64_t ldp_out, int64_t stride_p, void* stream) {
  if (m < 0 || n < 0 || ldp_bytes <= 0 || ldp_bytes % 32 != 0) return OZK_EINVAL;
  if (2 * ldp_bytes > round_up(OZK_MAX_K, kPlaneK)) return OZK_ERANGE;
  if (stride_a < m * ldp_bytes || stride_b < n * ldp_bytes || stride_a % 16 || stride_b % 16)
    return OZK_EINVAL;
  if (ldp_out < (n > 0 ? n : 1) || stride_p < m * ldp_out) return OZK_EINVAL;
  if (m == 0 || n == 0) return OZK_OK;
  if (!planes_a || !planes_b || !products || !aligned(planes_a, 16) || !aligned(planes_b, 16))
    return OZK_EINVAL;
  return launch_fp4_products(m, n, ldp_bytes, planes_a, stride_a, planes_b, stride_b, products,
                             ldp_out, stride_p, as_stream(stream));
}

int ozk_int8gemm_fp4limb_workspace_size(int64_t m, int64_t n, int64_t k, size_t* bytes) {
  if (!bytes || m < 0 || n < 0 || k < 1) return OZK_EINVAL;
  if (k > OZK_MAX_K) return OZK_ERANGE;
  const int64_t ldpb = round_up(k, 2 * kPlaneK) / 2;  // K steps of 128 codes
  *bytes = align256((size_t)3 * m * ldpb) + align256((size_t)3 * n * ldpb);
  return OZK_OK;
}

int ozk_int8gemm_fp4limb(int64_t m, int64_t n, int64_t k, const int8_t* A, int64_t lda,
                         const int8_t* B, int64_t ldb, int32_t* C, int64_t ldc, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (m < 0 || n < 0 || k < 1) return OZK_EINVAL;
  if (k > OZK_MAX_K) return OZK_ERANGE;
  if (lda < k || ldb < (n > 0 ? n : 1) || ldc < (n > 0 ? n : 1)) return OZK_EINVAL;
  if (m == 0 || n == 0) return OZK_OK;
  if (!A || !B || !C) return OZK_EINVAL;
  size_t need = 0;
  ozk_int8gemm_fp4limb_workspace_size(m, n, k, &need);
  if (!workspace || workspace_bytes < need) return OZK_EWORKSPACE;
  if (!aligned(workspace, 256)) return OZK_EINVAL;
  const int64_t ldpb = round_up(k, 2 * kPlaneK) / 2;  // K steps of 128 codes
  Carver cv(workspace);
  uint8_t* pa = static_cast<uint8_t*>(cv.take((size_t)3 * m * ldpb));
  uint8_t* pb = static_cast<uint8_t*>(cv.take((size_t)3 * n * ldpb));
  hipStream_t s = as_stream(stream);
  int st;
  if ((st = launch_fp4_pack(A, m, k, lda, 0, pa, ldpb, m * ldpb, s))) return st;
  if ((st = launch_fp4_pack(B, k, n, ldb, 1, pb, ldpb, n * ldpb, s))) return st;
  return launch_fp4_gemm(m, n, ldpb, pa, m * ldpb, pb, n * ldpb, C, ldc, s);
}

// ---------------------------------------------------------------- 6-product FP4 INT8 GEMM
int64_t ozk_fp4awe_line_bytes(int64_t k) { return k <= 0 ? 0 : awe_line_bytes(k); }

int ozk_fp4awe_pack(const int8_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                    uint8_t* planes, int64_t ld_line, void* stream) {
  if (axis != 0 && axis != 1) return OZK_EINVAL;
  if (rows < 0 || cols < 0 || ldx < (cols > 0 ? cols : 1)) return OZK_EINVAL;
  const int64_t K = axis == 0 ? cols : rows;
  const int64_t lines = axis == 0 ? rows : cols;
  if (K > OZK_MAX_K) return OZK_ERANGE;
  if (ld_line < awe_line_bytes(K > 0 ? K : 1) || ld_line % 16 != 0) return OZK_EINVAL;
  if (lines == 0 || K == 0) return OZK_OK;
  if (!planes || !x || !aligned(planes, 16)) return OZK_EINVAL;
  return launch_awe_pack(x, rows, cols, ldx, axis, planes, ld_line, as_stream(stream));
}

int ozk_fp4awe_products(int64_t m, int64_t n, int64_t k, const uint8_t* planes_a, int64_t lda,
                        const uint8_t* planes_b, int64_t ldb, int32_t* products,
                        int64_t ldp_out, int64_t stride_p, void* stream) {
  if (m < 0 || n < 0 || k < 1) return OZK_EINVAL;
  if (k > OZK_MAX_K) return OZK_ERANGE;
  const int64_t line = awe_line_bytes(k);
  if (lda < line || ldb < line || lda % 16 || ldb % 16) return OZK_EINVAL;
  if (ldp_out < (n > 0 ? n : 1) || stride_p < m * ldp_out) return OZK_EINVAL;
  if (m == 0 || n == 0) return OZK_OK;
  if (!planes_a || !planes_b || !products || !aligned(planes_a, 16) || !aligned(planes_b, 16))
    return OZK_EINVAL;
  return launch_awe_products(m, n, line / 192, planes_a, lda, planes_b, ldb, products, ldp_out,
                             stride_p, as_stream(stream));
}

int ozk_int8gemm_fp4awe_workspace_size(int64_t m, int64_t n, int64_t k, size_t* bytes) {
  if (!bytes || m < 0 || n < 0 || k < 1) return OZK_EINVAL;
  if (k > OZK_MAX_K) return OZK_ERANGE;
  const int64_t line = awe_line_bytes(k);
  *bytes = align256((size_t)m * line) + align256((size_t)n * line);
  return OZK_OK;
}

int ozk_int8gemm_fp4awe(int64_t m, int64_t n, int64_t k, const int8_t* A, int64_t lda,
                        const int8_t* B, int64_t ldb, int32_t* C, int64_t ldc, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (m < 0 || n < 0 || k < 1) return OZK_EINVAL;
  if (k > OZK_MAX_K) return OZK_ERANGE;
  if (lda < k || ldb < (n > 0 ? n : 1) || ldc < (n > 0 ? n : 1)) return OZK_EINVAL;
  if (m == 0 || n == 0) return OZK_OK;
  if (!A || !B || !C) return OZK_EINVAL;
  size_t need = 0;
  ozk_int8gemm_fp4awe_workspace_size(m, n, k, &need);
  if (!workspace || workspace_bytes < need) return OZK_EWORKSPACE;
  if (!aligned(workspace, 256)) return OZK_EINVAL;
  const int64_t line = awe_line_bytes(k);
  Carver cv(workspace);
  uint8_t* pa = static_cast<uint8_t*>(cv.take((size_t)m * line));
  uint8_t* pb = static_cast<uint8_t*>(cv.take((size_t)n * line));
  hipStream_t s = as_stream(stream);
  int st;
  if ((st = launch_awe_pack(A, m, k, lda, 0, pa, line, s))) return st;
  if ((st = launch_awe_pack(B, k, n, ldb, 1, pb, line, s))) return st;
  return launch_awe_gemm(m, n, line / 192, pa, line, pb, line, C, ldc, s);
}

// ---------------------------------------------------------------- 4-product FP4 INT4 x INT8 GEMM
int64_t ozk_fp4awe4_line_bytes(int64_t k) { return k <= 0 ? 0 : awe4_line_bytes(k); }

int ozk_fp4awe4_pack(const int8_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                     int int4, uint8_t* planes, int64_t ld_line, void* stream) {
  if (axis != 0 && axis != 1) return OZK_EINVAL;
  if (int4 != 0 && int4 != 1) return OZK_EINVAL;
  if (rows < 0 || cols < 0 || ldx < (cols > 0 ? cols : 1)) return OZK_EINVAL;
  const int64_t K = axis == 0 ? cols : rows;
  const int64_t lines = axis == 0 ? rows : cols;
  if (K > OZK_MAX_K) return OZK_ERANGE;
  if (ld_line < awe4_line_bytes(K > 0 ? K : 1) || ld_line % 16 != 0) return OZK_EINVAL;
  if (lines == 0 || K == 0) return OZK_OK;
  if (!planes || !x || !aligned(planes, 16)) return OZK_EINVAL;
  return launch_awe4_pack(x, rows, cols, ldx, axis, int4, planes, ld_line, as_stream(stream));
}

int ozk_fp4awe4_products(int64_t m, int64_t n, int64_t k, const uint8_t* planes_a,
                         int64_t lda, const uint8_t* planes_b, int64_t ldb, int32_t* products,
                         int64_t ldp_out, int64_t stride_p, void* stream) {
  if (m < 0 || n < 0 || k < 1) return OZK_EINVAL;
  if (k > OZK_MAX_K) return OZK_ERANGE;
  const int64_t line = awe4_line_bytes(k);
  if (lda < line || ldb < line || lda % 16 || ldb % 16) return OZK_EINVAL;
  if (ldp_out < (n > 0 ? n : 1) || stride_p < m * ldp_out) return OZK_EINVAL;
  if (m == 0 || n == 0) return OZK_OK;
  if (!planes_a || !planes_b || !products || !aligned(planes_a, 16) || !aligned(planes_b, 16))
    return OZK_EINVAL;
  return launch_awe4_products(m, n, line / 128, planes_a, lda, planes_b, ldb, products,
                              ldp_out, stride_p, as_stream(stream));
}

int ozk_int4int8gemm_fp4awe_workspace_size(int64_t m, int64_t n, int64_t k, size_t* bytes) {
  if (!bytes || m < 0 || n < 0 || k < 1) return OZK_EINVAL;
  if (k > OZK_MAX_K) return OZK_ERANGE;
  const int64_t line = awe4_line_bytes(k);
  *bytes = align256((size_t)m * line) + align256((size_t)n * line);
  return OZK_OK;
}

int ozk_int4int8gemm_fp4awe(int64_t m, int64_t n, int64_t k, const int8_t* A, int64_t lda,
                            const int8_t* B, int64_t ldb, int32_t* C, int64_t ldc,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (m < 0 || n < 0 || k < 1) return OZK_EINVAL;
  if (k > OZK_MAX_K) return OZK_ERANGE;
  if (lda < k || ldb < (n > 0 ? n : 1) || ldc < (n > 0 ? n : 1)) return OZK_EINVAL;
  if (m == 0 || n == 0) return OZK_OK;
  if (!A || !B || !C) return OZK_EINVAL;
  size_t need = 0;
  ozk_int4int8gemm_fp4awe_workspace_size(m, n, k, &need);
  if (!workspace || workspace_bytes < need) return OZK_EWORKSPACE;
  if (!aligned(workspace, 256)) return OZK_EINVAL;
  const int64_t line = awe4_line_bytes(k);
  Carver cv(workspace);
  uint8_t* pa = static_cast<uint8_t*>(cv.take((size_t)m * line));
  uint8_t* pb = static_cast<uint8_t*>(cv.take((size_t)n * line));
  hipStream_t s = as_stream(stream);
  int st;
  if ((st = launch_awe4_pack(A, m, k, lda, 0, 1, pa, line, s))) return st;
  if ((st = launch_awe4_pack(B, k, n, ldb, 1, 0, pb, line, s))) return st;
  return launch_awe4_gemm(m, n, line / 128, pa, line, pb, line, C, ldc, s);
}

}  // extern "C"

// ---------------------------------------------------------------- emulated SpMV (CSR)
namespace {

struct SpmvLayout {
  size_t x_res, x_exp, x_partial, res, row_exps;
  size_t total() const {
    return align256(x_res) + align256(x_exp) + align256(x_partial) + align256(res) +
           align256(row_exps);
  }
};

SpmvLayout spmv_layout(int64_t rows, int64_t cols, int r) {
  SpmvLayout L;
  L.x_res = (size_t)cols * (r <= 16 ? 16 : 32);
  L.x_exp = 4;
  L.x_partial = (size_t)((cols + 2047) / 2048) * 8;
  L.res = (size_t)r * rows;
  L.row_exps = (size_t)rows * 4;
  return L;
}

}  // namespace

extern "C" {

int ozk_spmv_csr_workspace_size(int64_t rows, int64_t cols, int r, size_t* bytes) {
  if (!bytes || rows < 0 || cols < 1 || check_r(r) != OZK_OK) return OZK_EINVAL;
  *bytes = spmv_layout(rows, cols, r).total();
  return OZK_OK;
}

int ozk_spmv_csr(int64_t rows, int64_t cols, int64_t nnz, const int32_t* row_ptr,
                 const int32_t* col_idx, const double* vals, int64_t max_row_nnz,
                 const double* x, double* y, int r, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (check_r(r) != OZK_OK) return OZK_EINVAL;
  if (rows < 0 || cols < 1 || nnz < 0 || max_row_nnz < 1) return OZK_EINVAL;
  if (nnz > 0x7fffffffll || rows > 0x7ffffffell || cols > 0x7fffffffll) return OZK_EUNSUPPORTED;
  if (max_row_nnz > OZK_MAX_K) return OZK_ERANGE;
  int pa = 0, pb = 0;
  int st = scaling_bits(r, max_row_nnz, &pa, &pb);
  if (st != OZK_OK) return st;
  if (rows == 0) return OZK_OK;
  if (!row_ptr || !x || !y || (nnz > 0 && (!col_idx || !vals))) return OZK_EINVAL;
  const SpmvLayout L = spmv_layout(rows, cols, r);
  if (!workspace || workspace_bytes < L.total()) return OZK_EWORKSPACE;
  if (!aligned(workspace, 256)) return OZK_EINVAL;
  Carver cv(workspace);
  int8_t* x_res = static_cast<int8_t*>(cv.take(L.x_res));
  int32_t* x_exp = static_cast<int32_t*>(cv.take(L.x_exp));
  uint64_t* x_partial = static_cast<uint64_t*>(cv.take(L.x_partial));
  int8_t* res = static_cast<int8_t*>(cv.take(L.res));
  int32_t* row_exps = static_cast<int32_t*>(cv.take(L.row_exps));
  hipStream_t s = as_stream(stream);
  if ((st = launch_spmv(rows, cols, nnz, row_ptr, col_idx, vals, max_row_nnz, x, r, pa, pb,
                        x_partial, x_exp, x_res, res, row_exps, s)))
    return st;
  // y as a 1 x rows matrix: output j scaled by x's exponent plus row j's
  return launch_crt(1, rows, r, res, 0, rows, rows, x_exp, row_exps, y, rows, s);
}

}  // extern "C"
