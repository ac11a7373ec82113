// Emulated sparse matrix-vector product y = A x, A in CSR: [TME4] abstract names sparse
// matrix-vector products among the memory-bound kernels whose emulation pays the
// per-input deconstruction term.  The arithmetic is the dense path's: rows of A scaled
// by the max rule over their nonzeros with the budget of dot products of at most kmax
// terms, x by one exponent, exact int32 row sums per modulus, CRT lift and one rounding
// (the CRT kernel of the dense path, on y as a 1 x rows matrix).
//
// x: its exponent from chunk maxima (no atomics) and one combining block, then its r
// residues per entry interleaved as xres[j][kXS] (16 bytes for r <= 16, else 32), so
// that a row entry gathers all of them with one or two 16-byte loads.
// spmv_residues_kernel: one thread per row, the workgroup's entries staged in LDS by
// coalesced loads.  The row's values are read twice (maximum, then residues), their
// residues are formed in registers, multiplied by the gathered residues of x and summed
// per modulus; the sums' symmetric residues go out as bytes [r][rows].  The row pass is
// instantiated per r, its moduli's constants compile-time values.  A row whose extent in
// row_ptr is not inside [0, nnz], that is longer than kmax or that holds a column index
// outside [0, cols) reads nothing through it and gets the exponent INT32_MIN (its y is
// NaN).
#include <type_traits>

#include "ozk_internal.h"
#include "residue_math.h"
#include "rns_table.h"

namespace ozk {
namespace {

// Low byte of the symmetric residue of an exact int32 sum v modulo an odd m <= 255 (q =
// round(v / m) from v * RN(1/m) + 1.5 * 2^52: within 2^-30 of v / m, whose distance to
// a half-integer is at least 1 / (2m), so the rounding is exact).
__device__ __forceinline__ uint32_t sum_residue_byte(int v, uint32_t m, double inv) {
  constexpr double kMagicD = 6755399441055744.0;
  const int q = (int)(uint32_t)__double_as_longlong(__builtin_fma((double)v, inv, kMagicD));
  return (uint32_t)(__mul24(q, -(int)m) + v);   // low byte: the low 24 bits of q suffice
}

// Largest |x| (bit pattern) of each chunk of 2048 entries.
__global__ __launch_bounds__(256) void vec_absmax_kernel(const double* __restrict__ x, int64_t n,
                                                         uint64_t* __restrict__ partial) {
  const int64_t base = (int64_t)blockIdx.x * 2048;
  uint64_t v = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t j = base + u * 256 + threadIdx.x;
    if (j < n) {
      const uint64_t b = abs_bits(x[j]);
      v = v > b ? v : b;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  __shared__ uint64_t w[4];
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t m = w[0];
    for (int q = 1; q < 4; ++q) m = m > w[q] ? m : w[q];
    partial[blockIdx.x] = m;
  }
}

// One block: the maximum over the chunk maxima, then x's max-rule exponent.
__global__ __launch_bounds__(256) void vec_exp_kernel(const uint64_t* __restrict__ partial,
                                                      int64_t chunks, int p_bits,
                                                      int32_t* __restrict__ exp) {
  uint64_t v = 0;
  for (int64_t c = threadIdx.x; c < chunks; c += 256) v = v > partial[c] ? v : partial[c];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  __shared__ uint64_t w[4];
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t m = w[0];
    for (int q = 1; q < 4; ++q) m = m > w[q] ? m : w[q];
    exp[0] = line_exponent(m, p_bits);
  }
}

// xres[j][0 .. kXS) = the r residues of x_j (zero past r, all zero if x's exponent marks
// Inf/NaN).
template <bool kWide, int kXS>
__global__ __launch_bounds__(256) void x_residues_kernel(const double* __restrict__ x, int64_t n,
                                                         const int32_t* __restrict__ exp,
                                                         ResidueConsts K,
                                                         int8_t* __restrict__ xres) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const int e0 = exp[0];
  const bool bad = e0 == INT32_MIN;
  const Prepared pr = prepare_element<kWide>(bad ? 0.0 : x[j], bad ? 0 : e0);
  uint32_t w[kXS / 4];
#pragma unroll
  for (int q = 0; q < kXS / 4; ++q) w[q] = 0;
  w[0] = residue_byte_256(pr) & 0xffu;
#pragma unroll
  for (int l = 1; l < kXS; ++l)
    if (l < K.r)
      w[l / 4] |= (residue_byte<kWide>(pr, K.m[l], K.inv[l], K.c32[l]) & 0xffu) << (8 * (l % 4));
  uint4* dst = reinterpret_cast<uint4*>(xres + j * kXS);
#pragma unroll
  for (int q = 0; q < kXS / 16; ++q)
    dst[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
}

// Moduli and their residue constants at compile time: the row pass is instantiated per r,
// so every modulus's constants are immediates or scalar moves and no per-modulus branch
// remains.
constexpr RnsTable kRns = make_rns_table();

template <int L, int N, typename F>
__device__ __forceinline__ void for_moduli(F&& f) {
  if constexpr (L < N) {
    f(std::integral_constant<int, L>{});
    for_moduli<L + 1, N>(f);
  }
}

constexpr int kSpmvRows = 256;    // rows (one per thread) per workgroup
constexpr int kSpmvCap = 2048;    // entries of a workgroup's rows staged in LDS

// One thread per row.  The workgroup first copies the values and column indices of its
// 256 rows (one contiguous range of the CSR arrays) into LDS with coalesced loads, when
// the range is well formed and holds at most kSpmvCap entries; a row then reads its
// entries from LDS if its extent lies inside that range, else from global memory (the
// result is the same either way).
template <bool kWide, int R>
__global__ __launch_bounds__(kSpmvRows) void spmv_residues_kernel(
    int64_t rows, int64_t cols, int64_t nnz, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, const double* __restrict__ vals, int64_t kmax,
    int p_bits, const int8_t* __restrict__ xres, int8_t* __restrict__ res,
    int32_t* __restrict__ exps) {
  constexpr int kXS = R <= 16 ? 16 : 32;     // bytes of x's residues per entry
  __shared__ double s_val[kSpmvCap];
  __shared__ int32_t s_col[kSpmvCap];
  const int64_t b0 = (int64_t)blockIdx.x * kSpmvRows;
  const int64_t bend = b0 + kSpmvRows < rows ? b0 + kSpmvRows : rows;
  const int64_t s0 = row_ptr[b0], s1 = row_ptr[bend];
  const bool staged = s0 >= 0 && s1 >= s0 && s1 <= nnz && s1 - s0 <= kSpmvCap;
  if (staged) {
    const int cnt = (int)(s1 - s0);
    for (int e = threadIdx.x; e < cnt; e += kSpmvRows) {
      s_val[e] = vals[s0 + e];
      s_col[e] = col_idx[s0 + e];
    }
  }
  __syncthreads();
  const int64_t i = b0 + threadIdx.x;
  if (i >= rows) return;
  const int64_t s = row_ptr[i], t = row_ptr[i + 1];

  auto row = [&](auto val_at, auto col_at) {
    bool ok = s >= 0 && t >= s && t <= nnz && t - s <= kmax;
    uint64_t mx = 0;
    if (ok) {
      for (int64_t p = s; p < t; ++p) {
        const int64_t c = col_at(p);
        ok = ok && c >= 0 && c < cols;
        const uint64_t b = abs_bits(val_at(p));
        mx = mx > b ? mx : b;
      }
    }
    const int e = ok ? line_exponent(mx, p_bits) : INT32_MIN;
    exps[i] = e;
    int acc[R];
#pragma unroll
    for (int l = 0; l < R; ++l) acc[l] = 0;
    if (e != INT32_MIN) {
      for (int64_t p = s; p < t; ++p) {
        const uint4* xs = reinterpret_cast<const uint4*>(xres + col_at(p) * kXS);
        uint32_t xw[kXS / 4];
#pragma unroll
        for (int q = 0; q < kXS / 16; ++q) {
          const uint4 v = xs[q];
          xw[4 * q] = v.x;
          xw[4 * q + 1] = v.y;
          xw[4 * q + 2] = v.z;
          xw[4 * q + 3] = v.w;
        }
        const Prepared pr = prepare_element<kWide>(val_at(p), e);
        acc[0] += (int)(int8_t)residue_byte_256(pr) * (int)(int8_t)(xw[0] & 0xffu);
        for_moduli<1, R>([&](auto lc) {
          constexpr int l = decltype(lc)::value;
          constexpr double m = (double)kRns.moduli[l], inv = kRns.inv[l], c32 = kRns.c32[l];
          acc[l] += (int)(int8_t)residue_byte<kWide>(pr, m, inv, c32) *
                    (int)(int8_t)((xw[l / 4] >> (8 * (l % 4))) & 0xffu);
        });
      }
    }
    res[i] = (int8_t)(acc[0] & 0xff);
    for_moduli<1, R>([&](auto lc) {
      constexpr int l = decltype(lc)::value;
      constexpr uint32_t m = (uint32_t)kRns.moduli[l];
      constexpr double inv = kRns.inv[l];
      res[l * rows + i] = (int8_t)sum_residue_byte(acc[l], m, inv);
    });
  };
  if (staged && s >= s0 && t >= s && t <= s1)
    row([&](int64_t p) { return s_val[p - s0]; }, [&](int64_t p) { return (int64_t)s_col[p - s0]; });
  else
    row([&](int64_t p) { return vals[p]; }, [&](int64_t p) { return (int64_t)col_idx[p]; });
}

template <int... Rs>
struct SpmvDispatch {
  static void go(int, bool, dim3, hipStream_t, int64_t, int64_t, int64_t, const int32_t*,
                 const int32_t*, const double*, int64_t, int, const int8_t*, int8_t*, int32_t*) {}
};

template <int R0, int... Rs>
struct SpmvDispatch<R0, Rs...> {
  static void go(int r, bool wide, dim3 g, hipStream_t s, int64_t rows, int64_t cols,
                 int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx, const double* vals,
                 int64_t kmax, int p_a, const int8_t* xres, int8_t* res, int32_t* exps) {
    if (r != R0) {
      SpmvDispatch<Rs...>::go(r, wide, g, s, rows, cols, nnz, row_ptr, col_idx, vals, kmax, p_a,
                              xres, res, exps);
    } else if (wide) {
      hipLaunchKernelGGL((spmv_residues_kernel<true, R0>), g, dim3(kSpmvRows), 0, s, rows, cols,
                         nnz, row_ptr, col_idx, vals, kmax, p_a, xres, res, exps);
    } else {
      hipLaunchKernelGGL((spmv_residues_kernel<false, R0>), g, dim3(kSpmvRows), 0, s, rows, cols,
                         nnz, row_ptr, col_idx, vals, kmax, p_a, xres, res, exps);
    }
  }
};

}  // namespace

int launch_spmv(int64_t rows, int64_t cols, int64_t nnz, const int32_t* row_ptr,
                const int32_t* col_idx, const double* vals, int64_t kmax, const double* x,
                int r, int p_a, int p_b, uint64_t* x_partial, int32_t* x_exp, int8_t* xres,
                int8_t* res, int32_t* exps, hipStream_t s) {
  if (rows <= 0) return OZK_OK;
  if (!residue_consts(r, p_b) || !residue_consts(r, p_a)) return OZK_EINVAL;
  const int64_t chunks = (cols + 2047) / 2048;
  hipLaunchKernelGGL(vec_absmax_kernel, dim3((unsigned)chunks), dim3(256), 0, s, x, cols,
                     x_partial);
  hipLaunchKernelGGL(vec_exp_kernel, dim3(1), dim3(256), 0, s, x_partial, chunks, p_b, x_exp);
  if (hipGetLastError() != hipSuccess) return OZK_EHIP;
  const ResidueConsts& KB = *residue_consts(r, p_b);
  const ResidueConsts& KA = *residue_consts(r, p_a);
  const dim3 gx((unsigned)((cols + 255) / 256)), gr((unsigned)((rows + kSpmvRows - 1) / kSpmvRows));
  // one residue arithmetic for both sides: the wide one if either side needs it
  const bool wide = KA.wide || KB.wide;
  if (r <= 16) {
    if (wide)
      hipLaunchKernelGGL((x_residues_kernel<true, 16>), gx, dim3(256), 0, s, x, cols, x_exp, KB,
                         xres);
    else
      hipLaunchKernelGGL((x_residues_kernel<false, 16>), gx, dim3(256), 0, s, x, cols, x_exp,
                         KB, xres);
  } else {
    if (wide)
      hipLaunchKernelGGL((x_residues_kernel<true, 32>), gx, dim3(256), 0, s, x, cols, x_exp, KB,
                         xres);
    else
      hipLaunchKernelGGL((x_residues_kernel<false, 32>), gx, dim3(256), 0, s, x, cols, x_exp,
                         KB, xres);
  }
  SpmvDispatch<1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20>::go(
      r, wide, gr, s, rows, cols, nnz, row_ptr, col_idx, vals, kmax, p_a, xres, res, exps);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

}  // namespace ozk
