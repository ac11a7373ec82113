// Emulated sparse matrix-vector product y = A x, A in CSR: [TME4] abstract names sparse
// matrix-vector products among the memory-bound kernels whose emulation pays the
// per-input deconstruction term.  The arithmetic is the dense path's: rows of A scaled
// by the max rule over their nonzeros with the budget of dot products of at most kmax
// terms, x by one exponent (its residue planes come from the row deconstruction of x
// as a 1 x n matrix), exact int32 row sums per modulus, CRT lift and one rounding (the
// CRT kernel of the dense path, on y as a 1 x rows matrix).
//
// spmv_residues_kernel: one thread per row.  The row's values are read twice (maximum,
// then residues; the second read hits the cache), their residues are formed in
// registers, multiplied by the gathered residues of x and summed per modulus; the sums'
// symmetric residues go out as bytes [r][rows].  A row whose extent in row_ptr is not
// inside [0, nnz], that is longer than kmax or that holds a column index outside
// [0, cols) reads nothing through it and gets the exponent INT32_MIN (its y is NaN).
#include "ozk_internal.h"
#include "residue_math.h"

namespace ozk {
namespace {

// Low byte of the symmetric residue of an exact int32 sum v modulo an odd m <= 255 (q =
// round(v / m) from v * RN(1/m) + 1.5 * 2^52: within 2^-30 of v / m, whose distance to
// a half-integer is at least 1 / (2m), so the rounding is exact).
__device__ __forceinline__ uint32_t sum_residue_byte(int v, uint32_t m, double inv) {
  constexpr double kMagicD = 6755399441055744.0;
  const uint32_t q = (uint32_t)__double_as_longlong(__builtin_fma((double)v, inv, kMagicD));
  return (uint32_t)v - __umul24(q, m);
}

template <bool kWide>
__global__ __launch_bounds__(256) void spmv_residues_kernel(
    int64_t rows, int64_t cols, int64_t nnz, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, const double* __restrict__ vals, int64_t kmax,
    ResidueConsts K, int p_bits, const int8_t* __restrict__ xres, int64_t x_stride,
    int8_t* __restrict__ res, int32_t* __restrict__ exps) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows) return;
  const int64_t s = row_ptr[i], t = row_ptr[i + 1];
  bool ok = s >= 0 && t >= s && t <= nnz && t - s <= kmax;
  uint64_t mx = 0;
  if (ok) {
    for (int64_t p = s; p < t; ++p) {
      const int64_t c = col_idx[p];
      ok = ok && c >= 0 && c < cols;
      mx = mx > abs_bits(vals[p]) ? mx : abs_bits(vals[p]);
    }
  }
  int e = ok ? line_exponent(mx, p_bits) : INT32_MIN;
  exps[i] = e;
  int acc[kMaxModuli];
#pragma unroll
  for (int l = 0; l < kMaxModuli; ++l) acc[l] = 0;
  if (e != INT32_MIN) {
    for (int64_t p = s; p < t; ++p) {
      const int64_t c = col_idx[p];
      const Prepared pr = prepare_element<kWide>(vals[p], e);
      acc[0] += (int)(int8_t)residue_byte_256(pr) * (int)xres[c];
#pragma unroll
      for (int l = 1; l < kMaxModuli; ++l)
        if (l < K.r)
          acc[l] += (int)(int8_t)residue_byte<kWide>(pr, K.m[l], K.inv[l], K.c32[l]) *
                    (int)xres[l * x_stride + c];
    }
  }
  res[i] = (int8_t)(acc[0] & 0xff);
#pragma unroll
  for (int l = 1; l < kMaxModuli; ++l)
    if (l < K.r)
      res[l * rows + i] = (int8_t)sum_residue_byte(acc[l], (uint32_t)K.m[l], K.inv[l]);
}

}  // namespace

int launch_spmv_residues(int64_t rows, int64_t cols, int64_t nnz, const int32_t* row_ptr,
                         const int32_t* col_idx, const double* vals, int64_t kmax, int r,
                         int p_bits, const int8_t* xres, int64_t x_stride, int8_t* res,
                         int32_t* exps, hipStream_t s) {
  if (rows <= 0) return OZK_OK;
  const ResidueConsts& K = *residue_consts(r, p_bits);
  const dim3 grid((unsigned)((rows + 255) / 256));
  if (K.wide)
    hipLaunchKernelGGL(spmv_residues_kernel<true>, grid, dim3(256), 0, s, rows, cols, nnz,
                       row_ptr, col_idx, vals, kmax, K, p_bits, xres, x_stride, res, exps);
  else
    hipLaunchKernelGGL(spmv_residues_kernel<false>, grid, dim3(256), 0, s, rows, cols, nnz,
                       row_ptr, col_idx, vals, kmax, K, p_bits, xres, x_stride, res, exps);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

}  // namespace ozk
