// Deconstruction kernels: per-line exponents by the max rule and the r int8 residue
// planes, written K-contiguous.  [TME4] abstract (the per-input deconstruction term).
//
// Kernels
//   fill_u64            clears the column-maximum scratch before atomics
//   absmax_rows/cols    bit pattern of max |x| per row / column (atomicMax on u64;
//                       the order of non-negative doubles equals that of their bits,
//                       and Inf/NaN patterns sort above every finite value)
//   residues_rows       8 consecutive K elements per thread -> 8 bytes per plane
//   residues_cols       16 consecutive K elements of one column per thread -> 16 bytes
//                       per plane, 8 threads per 128-byte plane line (the transpose
//                       happens in the store address)
//   residues_rows_fused one workgroup per row: the row is held in registers, reduced
//                       for its maximum (and, by the norm rule, for its scaled sum of
//                       squares), then turned into residues (one HBM read)
//   norm_partials_rows/cols  norm rule: per chunk of a line, its maximum and its sum of
//                       squares scaled by that maximum's power of two
//   exps_norm           norm rule: chunk partials combined in order, exponent per line
#include "ozk_internal.h"
#include "residue_math.h"

namespace ozk {
namespace {

__global__ void fill_u64_kernel(uint64_t* __restrict__ p, int64_t n, uint64_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint64_t o = __shfl_xor(v, off, 64);
    v = umax64(v, o);
  }
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Row maxima: grid (chunks of 2048 columns, rows); 256 threads x 8 elements.
__global__ __launch_bounds__(256) void absmax_rows_kernel(const double* __restrict__ x,
                                                          int64_t cols, int64_t ldx,
                                                          uint64_t* __restrict__ maxbits) {
  const int64_t row = blockIdx.y;
  const int64_t base = (int64_t)blockIdx.x * 2048;
  const double* xr = x + row * ldx;
  uint64_t v = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    int64_t h = base + u * 256 + threadIdx.x;
    if (h < cols) v = umax64(v, abs_bits(xr[h]));
  }
  v = wave_max_u64(v);
  __shared__ uint64_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t m = umax64(umax64(part[0], part[1]), umax64(part[2], part[3]));
    atomicMax((unsigned long long*)&maxbits[row], (unsigned long long)m);
  }
}

// Column maxima: grid (column blocks of 256, row chunks of 64).
__global__ __launch_bounds__(256) void absmax_cols_kernel(const double* __restrict__ x,
                                                          int64_t rows, int64_t cols,
                                                          int64_t ldx,
                                                          uint64_t* __restrict__ maxbits) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (col >= cols) return;
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  const int64_t r1 = r0 + 64 < rows ? r0 + 64 : rows;
  uint64_t v = 0;
#pragma unroll 16
  for (int64_t h = r0; h < r1; ++h) v = umax64(v, abs_bits(x[h * ldx + col]));
  atomicMax((unsigned long long*)&maxbits[col], (unsigned long long)v);
}

// Residues of kN (8 or 16) consecutive prepared elements for every modulus, stored as
// kN bytes per plane.
template <int kN>
struct Bytes;
template <>
struct Bytes<8> {
  typedef uint2 type;
};
template <>
struct Bytes<16> {
  typedef uint4 type;
};

template <bool kWide, int kN>
__device__ __forceinline__ void store_residues(const double (&a)[kN], int e,
                                               const ResidueConsts& K, int8_t* dst,
                                               int64_t plane_stride) {
  typedef typename Bytes<kN>::type V;
  Prepared p[kN];
#pragma unroll
  for (int u = 0; u < kN; ++u) p[u] = prepare_element<kWide>(a[u], e);
  {
    uint32_t w[kN / 4];
#pragma unroll
    for (int q = 0; q < kN / 4; ++q)
      w[q] = pack4(residue_byte_256(p[4 * q]), residue_byte_256(p[4 * q + 1]),
                   residue_byte_256(p[4 * q + 2]), residue_byte_256(p[4 * q + 3]));
    *reinterpret_cast<V*>(dst) = *reinterpret_cast<const V*>(w);
  }
  for (int l = 1; l < K.r; ++l) {
    const double m = K.m[l], inv = K.inv[l], c = K.c32[l];
    uint32_t b[kN];
#pragma unroll
    for (int u = 0; u < kN; ++u) b[u] = residue_byte<kWide>(p[u], m, inv, c);
    uint32_t w[kN / 4];
#pragma unroll
    for (int q = 0; q < kN / 4; ++q) w[q] = pack4(b[4 * q], b[4 * q + 1], b[4 * q + 2], b[4 * q + 3]);
    *reinterpret_cast<V*>(dst + l * plane_stride) = *reinterpret_cast<const V*>(w);
  }
}

// 8 consecutive elements x[h0 .. h0+7] (0 beyond cols), 16-byte loads when aligned.
template <bool kVec>
__device__ __forceinline__ void load8(const double* __restrict__ xr, int64_t h0, int64_t cols,
                                      double (&a)[8]) {
  if (kVec && h0 + 8 <= cols) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const double2 v = *reinterpret_cast<const double2*>(xr + h0 + 2 * u);
      a[2 * u] = v.x;
      a[2 * u + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = h0 + u < cols ? xr[h0 + u] : 0.0;
  }
}

// Row residues with exponents from maxbits: grid (ldp / 2048 chunks, rows).
// kGiven: the exponents are already in exps (norm rule); else the max rule from maxbits.
template <bool kWide, bool kVec, bool kGiven>
__global__ __launch_bounds__(256) void residues_rows_kernel(
    const double* __restrict__ x, int64_t cols, int64_t ldx, ResidueConsts K, int p_bits,
    const uint64_t* __restrict__ maxbits, int8_t* __restrict__ planes, int64_t ldp,
    int64_t plane_stride, int32_t* __restrict__ exps) {
  const int64_t row = blockIdx.y;
  const int e = kGiven ? exps[row] : line_exponent(maxbits[row], p_bits);
  if (!kGiven && blockIdx.x == 0 && threadIdx.x == 0) exps[row] = e;
  const int64_t h0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (h0 >= ldp) return;
  const double* xr = x + row * ldx;
  double a[8];
  load8<kVec>(xr, h0, e == INT32_MIN ? 0 : cols, a);
  int8_t* dst = planes + row * ldp + h0;
  store_residues<kWide, 8>(a, e == INT32_MIN ? 0 : e, K, dst, plane_stride);
}

// Column residues: grid (ceil(cols/32), ceil(ldp/128)).  Lane t of wave w owns column
// j0 + 8w + (t >> 3) and K rows h0 + 16*(t & 7) .. +15; the eight lanes of a column store
// one whole 128-byte line of each plane row (16 bytes each), and each load instruction
// reads 8 rows x 8 columns (the four waves of a block read the 32 columns of a row, so
// every line is fetched once).
// Block (bx, by) of the column residues: 32 columns x 128 K positions.
template <bool kWide, bool kGiven>
__device__ __forceinline__ void cols_block(
    int64_t bx, int64_t by, const double* __restrict__ x, int64_t rows, int64_t cols,
    int64_t ldx, const ResidueConsts& K, int p_bits, const uint64_t* __restrict__ maxbits,
    int8_t* __restrict__ planes, int64_t ldp, int64_t plane_stride,
    int32_t* __restrict__ exps) {
  const int64_t col = bx * 32 + (threadIdx.x >> 3);
  if (col >= cols) return;
  const int64_t h0 = by * 128 + (threadIdx.x & 7) * 16;
  if (h0 >= ldp) return;  // ldp is a multiple of 64: the last block row may be half full
  const int e = kGiven ? exps[col] : line_exponent(maxbits[col], p_bits);
  if (!kGiven && by == 0 && (threadIdx.x & 7) == 0) exps[col] = e;
  double a[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int64_t h = h0 + u;
    a[u] = (h < rows && e != INT32_MIN) ? x[h * ldx + col] : 0.0;
  }
  store_residues<kWide, 16>(a, e == INT32_MIN ? 0 : e, K, planes + col * ldp + h0, plane_stride);
}

template <bool kWide, bool kGiven>
__global__ __launch_bounds__(256) void residues_cols_kernel(
    const double* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, ResidueConsts K,
    int p_bits, const uint64_t* __restrict__ maxbits, int8_t* __restrict__ planes,
    int64_t ldp, int64_t plane_stride, int32_t* __restrict__ exps) {
  cols_block<kWide, kGiven>(blockIdx.x, blockIdx.y, x, rows, cols, ldx, K, p_bits, maxbits,
                            planes, ldp, plane_stride, exps);
}

// One workgroup per row, the row in registers: kNT threads x kG groups of 8 elements.
// `width` is P of the max rule, or alpha of the norm rule (kNorm).
template <bool kWide, bool kVec, int kNT, int kG, bool kNorm>
__device__ __forceinline__ void rows_fused_block(
    int64_t row, const double* __restrict__ x, int64_t cols, int64_t ldx,
    const ResidueConsts& K, int width, int8_t* __restrict__ planes, int64_t ldp,
    int64_t plane_stride, int32_t* __restrict__ exps) {
  const double* xr = x + row * ldx;
  double a[kG][8];
  uint64_t v = 0;
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const int64_t h0 = ((int64_t)g * kNT + threadIdx.x) * 8;
    load8<kVec>(xr, h0, cols, a[g]);
#pragma unroll
    for (int u = 0; u < 8; ++u) v = umax64(v, abs_bits(a[g][u]));
  }
  v = wave_max_u64(v);
  __shared__ uint64_t part[kNT / 64];
  __shared__ double psum[kNT / 64];
  __shared__ int exp_shared;
  __shared__ uint64_t max_shared;
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t mx = 0;
    for (int w = 0; w < kNT / 64; ++w) mx = umax64(mx, part[w]);
    if (kNorm) {
      max_shared = mx;
    } else {
      int e = line_exponent(mx, width);
      exp_shared = e;
      exps[row] = e;
    }
  }
  __syncthreads();
  if (kNorm) {
    // Sum of (x 2^-T)^2: per thread in element order, lanes by a fixed butterfly, waves
    // in order (deterministic).
    const uint64_t mx = max_shared;
    const int t = line_ilogb(mx);
    double ss = 0.0;
#pragma unroll
    for (int g = 0; g < kG; ++g)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const double y = __builtin_ldexp(a[g][u], -t);
        ss = __builtin_fma(y, y, ss);
      }
    ss = wave_sum_f64(ss);
    if ((threadIdx.x & 63) == 0) psum[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0) {
      double s = 0.0;
      for (int w = 0; w < kNT / 64; ++w) s += psum[w];
      const int e = norm_exponent(mx, s, width);
      exp_shared = e;
      exps[row] = e;
    }
    __syncthreads();
  }
  int e = exp_shared;
  const bool bad = e == INT32_MIN;
  if (bad) e = 0;
  int8_t* prow = planes + row * ldp;
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const int64_t h0 = ((int64_t)g * kNT + threadIdx.x) * 8;
    if (h0 >= ldp) continue;
    if (bad) {
#pragma unroll
      for (int u = 0; u < 8; ++u) a[g][u] = 0.0;
    }
    store_residues<kWide, 8>(a[g], e, K, prow + h0, plane_stride);
  }
  // Padding beyond the register-resident part (only when ldp exceeds kNT * kG * 8).
  for (int64_t h0 = ((int64_t)kG * kNT + threadIdx.x) * 8; h0 < ldp; h0 += (int64_t)kNT * 8) {
    for (int l = 0; l < K.r; ++l)
      *reinterpret_cast<uint2*>(prow + l * plane_stride + h0) = make_uint2(0u, 0u);
  }
}

template <bool kWide, bool kVec, int kNT, int kG, bool kNorm>
__global__ __launch_bounds__(kNT) void residues_rows_fused_kernel(
    const double* __restrict__ x, int64_t cols, int64_t ldx, ResidueConsts K, int width,
    int8_t* __restrict__ planes, int64_t ldp, int64_t plane_stride,
    int32_t* __restrict__ exps) {
  rows_fused_block<kWide, kVec, kNT, kG, kNorm>(blockIdx.x, x, cols, ldx, K, width, planes,
                                                ldp, plane_stride, exps);
}

// Both operands of a product in one launch: the rows of A (fused, one block per row)
// and the column residues of B (exponents or maxima of B already computed), their
// blocks interleaved so that the VALU-heavier row blocks and the store-heavier column
// blocks share the chip.  Block b < 2 min(nA, nB) takes A row b / 2 (even b) or B block
// b / 2 (odd b); the rest go to whichever operand has more.
struct PairArgs {
  const double* a;
  int64_t m, k, lda;
  ResidueConsts ka;
  int width_a;
  int8_t* planes_a;
  int32_t* exps_a;
  const double* b;
  int64_t n, ldb;
  ResidueConsts kb;
  int width_b;
  const uint64_t* maxbits_b;
  int8_t* planes_b;
  int32_t* exps_b;
  int64_t kp, gx_b, blocks_b;
};

template <bool kWide, bool kVec, int kG, bool kNorm>
__global__ __launch_bounds__(256) void deconstruct_pair_kernel(PairArgs p) {
  const int64_t b = blockIdx.x;
  const int64_t both = p.m < p.blocks_b ? p.m : p.blocks_b;
  bool is_a;
  int64_t idx;
  if (b < 2 * both) {
    is_a = (b & 1) == 0;
    idx = b >> 1;
  } else {
    is_a = p.m > p.blocks_b;
    idx = both + (b - 2 * both);
  }
  if (is_a)
    rows_fused_block<kWide, kVec, 256, kG, kNorm>(idx, p.a, p.k, p.lda, p.ka, p.width_a,
                                                  p.planes_a, p.kp, p.m * p.kp, p.exps_a);
  else
    cols_block<kWide, kNorm>(idx % p.gx_b, idx / p.gx_b, p.b, p.k, p.n, p.ldb, p.kb, p.width_b,
                             p.maxbits_b, p.planes_b, p.kp, p.n * p.kp, p.exps_b);
}

// Norm rule outside the fused kernel.  The line is cut into chunks; each chunk writes
// its own largest |x| (bit pattern) pmax and ps = sum of (x 2^-Tc)^2 with Tc = ilogb of
// that maximum, in a fixed order.  exps_norm_kernel then takes T = ilogb of the line's
// maximum and s = the chunks' ps 2^(2 (Tc - T)) added in a fixed order: scaling by a
// power of two is exact, so s is the line's scaled sum of squares in a fixed order
// (terms that underflow are below 2^-1000 of s >= 1, far inside the bound's slack).
// The line is read once for its exponent, as by the max rule.

// Rows: grid (chunks of 2048 columns, rows); 256 threads x 8 elements,
// written to pmax/ps[row * gridDim.x + chunk].
__global__ __launch_bounds__(256) void norm_partials_rows_kernel(
    const double* __restrict__ x, int64_t cols, int64_t ldx, uint64_t* __restrict__ pmax,
    double* __restrict__ ps) {
  const int64_t row = blockIdx.y;
  const int64_t base = (int64_t)blockIdx.x * 2048;
  const double* xr = x + row * ldx;
  double a[8];
  uint64_t v = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t h = base + u * 256 + threadIdx.x;
    a[u] = h < cols ? xr[h] : 0.0;
    v = umax64(v, abs_bits(a[u]));
  }
  v = wave_max_u64(v);
  __shared__ uint64_t wm[4];
  __shared__ double ws[4];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = v;
  __syncthreads();
  const uint64_t mx = umax64(umax64(wm[0], wm[1]), umax64(wm[2], wm[3]));
  const int t = line_ilogb(mx);
  double ss = 0.0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const double y = __builtin_ldexp(a[u], -t);
    ss = __builtin_fma(y, y, ss);
  }
  ss = wave_sum_f64(ss);
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t i = row * gridDim.x + blockIdx.x;
    pmax[i] = mx;
    ps[i] = ((ws[0] + ws[1]) + ws[2]) + ws[3];
  }
}

// Adds a piece (maximum mc, sum sc scaled by 2^-2Tc, Tc = ilogb mc) into a running
// (maximum m, sum s scaled by 2^-2T): both sums are brought to the larger maximum's
// exponent by exact power-of-two scalings, then added.
__device__ __forceinline__ void norm_combine(uint64_t& m, double& s, uint64_t mc, double sc) {
  const uint64_t mn = umax64(m, mc);
  const int t = line_ilogb(mn);
  s = __builtin_ldexp(s, 2 * (line_ilogb(m) - t)) + __builtin_ldexp(sc, 2 * (line_ilogb(mc) - t));
  m = mn;
}

// Columns: grid (column blocks of 256, chunks of 128 rows); thread = column.  The chunk
// is taken as 4 pieces of 32 rows held in registers (maximum, then scaled squares), the
// pieces combined in order; written to pmax/ps[chunk * cols + col].
__global__ __launch_bounds__(256) void norm_partials_cols_kernel(
    const double* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    uint64_t* __restrict__ pmax, double* __restrict__ ps) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (col >= cols) return;
  uint64_t m = 0;
  double s = 0.0;
  for (int piece = 0; piece < 4; ++piece) {
    const int64_t r0 = (int64_t)blockIdx.y * 128 + piece * 32;
    if (r0 >= rows) break;
    double a[32];
    uint64_t v = 0;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      a[u] = r0 + u < rows ? x[(r0 + u) * ldx + col] : 0.0;
      v = umax64(v, abs_bits(a[u]));
    }
    const int t = line_ilogb(v);
    double ss = 0.0;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const double y = __builtin_ldexp(a[u], -t);
      ss = __builtin_fma(y, y, ss);
    }
    norm_combine(m, s, v, ss);
  }
  const int64_t i = (int64_t)blockIdx.y * cols + col;
  pmax[i] = m;
  ps[i] = s;
}

// Per line: combine the chunk partials and write the norm-rule exponent.  Block of 256
// threads = 16 lines x 16 parts; part p combines chunks p, p + 16, ... in order, then
// the 16 parts are combined in order (deterministic).
__global__ __launch_bounds__(256) void exps_norm_kernel(
    const uint64_t* __restrict__ pmax, const double* __restrict__ ps, int64_t lines,
    int64_t chunks, int64_t stride_line, int64_t stride_chunk, int alpha,
    int32_t* __restrict__ exps) {
  const int j = threadIdx.x & 15, part = threadIdx.x >> 4;
  const int64_t i = (int64_t)blockIdx.x * 16 + j;
  uint64_t m = 0;
  double s = 0.0;
  if (i < lines)
    for (int64_t c = part; c < chunks; c += 16) {
      const int64_t q = i * stride_line + c * stride_chunk;
      norm_combine(m, s, pmax[q], ps[q]);
    }
  __shared__ uint64_t lm[16][17];
  __shared__ double ls[16][17];
  lm[j][part] = m;
  ls[j][part] = s;
  __syncthreads();
  if (part == 0 && i < lines) {
    uint64_t mm = 0;
    double sum = 0.0;
    for (int p = 0; p < 16; ++p) norm_combine(mm, sum, lm[j][p], ls[j][p]);
    exps[i] = norm_exponent(mm, sum, alpha);
  }
}

__global__ void exps_from_maxbits_kernel(const uint64_t* __restrict__ maxbits, int64_t n,
                                         int p_bits, int32_t* __restrict__ exps) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) exps[i] = line_exponent(maxbits[i], p_bits);
}

template <bool kWide, int kNT, int kG>
int launch_fused(const double* x, int64_t rows, int64_t cols, int64_t ldx,
                 const ResidueConsts& K, int norm, int width, int8_t* planes, int64_t ldp,
                 int64_t plane_stride, int32_t* exps, hipStream_t s) {
  const bool vec = (reinterpret_cast<uintptr_t>(x) & 15) == 0 && (ldx & 1) == 0;
#define OZK_FUSED_LAUNCH(V, N)                                                              \
  hipLaunchKernelGGL((residues_rows_fused_kernel<kWide, V, kNT, kG, N>), dim3((unsigned)rows), \
                     dim3(kNT), 0, s, x, cols, ldx, K, width, planes, ldp, plane_stride, exps)
  if (vec && norm) OZK_FUSED_LAUNCH(true, true);
  else if (vec) OZK_FUSED_LAUNCH(true, false);
  else if (norm) OZK_FUSED_LAUNCH(false, true);
  else OZK_FUSED_LAUNCH(false, false);
#undef OZK_FUSED_LAUNCH
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

}  // namespace

int launch_fill_u64(uint64_t* p, int64_t n, uint64_t v, hipStream_t s) {
  if (n <= 0) return OZK_OK;
  hipLaunchKernelGGL(fill_u64_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p,
                     n, v);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

int launch_absmax(const double* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                  uint64_t* maxbits, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return OZK_OK;
  if (axis == 0) {
    if (rows > 65535) return OZK_EUNSUPPORTED;
    dim3 grid((unsigned)((cols + 2047) / 2048), (unsigned)rows);
    hipLaunchKernelGGL(absmax_rows_kernel, grid, dim3(256), 0, s, x, cols, ldx, maxbits);
  } else {
    dim3 grid((unsigned)((cols + 255) / 256), (unsigned)((rows + 63) / 64));
    hipLaunchKernelGGL(absmax_cols_kernel, grid, dim3(256), 0, s, x, rows, cols, ldx, maxbits);
  }
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

int launch_residues(const double* x, int64_t rows, int64_t cols, int64_t ldx, int axis, int r,
                    int p_bits, const uint64_t* maxbits, int8_t* planes, int64_t ldp,
                    int64_t plane_stride, int32_t* exps, int given_exps, hipStream_t s) {
  if (!residue_consts(r, p_bits)) return OZK_EINVAL;
  const ResidueConsts& K = *residue_consts(r, p_bits);
  const bool wide = K.wide != 0;
  if (axis == 0) {
    if (rows <= 0) return OZK_OK;
    if (rows > 65535) return OZK_EUNSUPPORTED;
    dim3 grid((unsigned)((ldp + 2047) / 2048), (unsigned)rows);
    const bool vec = (reinterpret_cast<uintptr_t>(x) & 15) == 0 && (ldx & 1) == 0;
#define OZK_ROWS(W, V, G)                                                                     \
  hipLaunchKernelGGL((residues_rows_kernel<W, V, G>), grid, dim3(256), 0, s, x, cols, ldx, K, \
                     p_bits, maxbits, planes, ldp, plane_stride, exps)
#define OZK_ROWS_G(W, V) \
  if (given_exps) OZK_ROWS(W, V, true); else OZK_ROWS(W, V, false)
    if (wide && vec) { OZK_ROWS_G(true, true); }
    else if (wide) { OZK_ROWS_G(true, false); }
    else if (vec) { OZK_ROWS_G(false, true); }
    else { OZK_ROWS_G(false, false); }
#undef OZK_ROWS_G
#undef OZK_ROWS
  } else {
    if (cols <= 0) return OZK_OK;
    dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((ldp + 127) / 128));
#define OZK_COLS(W, G)                                                                      \
  hipLaunchKernelGGL((residues_cols_kernel<W, G>), grid, dim3(256), 0, s, x, rows, cols, ldx, \
                     K, p_bits, maxbits, planes, ldp, plane_stride, exps)
    if (wide && given_exps) OZK_COLS(true, true);
    else if (wide) OZK_COLS(true, false);
    else if (given_exps) OZK_COLS(false, true);
    else OZK_COLS(false, false);
#undef OZK_COLS
  }
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

bool rows_fused_supported(int64_t cols) { return cols <= 32768; }

int launch_deconstruct_pair(const double* a, int64_t m, int64_t k, int64_t lda, const double* b,
                            int64_t n, int64_t ldb, int r, int scaling, int width_a, int width_b,
                            const uint64_t* maxbits_b, int8_t* planes_a, int8_t* planes_b,
                            int64_t kp, int32_t* exps_a, int32_t* exps_b, hipStream_t s) {
  if (!residue_consts(r, width_a) || !residue_consts(r, width_b)) return OZK_EINVAL;
  const ResidueConsts& ka = *residue_consts(r, width_a);
  const ResidueConsts& kb = *residue_consts(r, width_b);
  if (ka.wide != kb.wide || k > 8192 || m <= 0 || n <= 0) return OZK_EUNSUPPORTED;
  PairArgs p;
  p.a = a; p.m = m; p.k = k; p.lda = lda; p.ka = ka; p.width_a = width_a;
  p.planes_a = planes_a; p.exps_a = exps_a;
  p.b = b; p.n = n; p.ldb = ldb; p.kb = kb; p.width_b = width_b; p.maxbits_b = maxbits_b;
  p.planes_b = planes_b; p.exps_b = exps_b; p.kp = kp;
  p.gx_b = (n + 31) / 32;
  p.blocks_b = p.gx_b * ((kp + 127) / 128);
  const int64_t blocks = m + p.blocks_b;
  if (blocks > 0x7fffffff) return OZK_EUNSUPPORTED;
  const bool vec = (reinterpret_cast<uintptr_t>(a) & 15) == 0 && (lda & 1) == 0;
  const bool norm = scaling == OZK_SCALING_NORM;
  const int g = k <= 2048 ? 1 : (k <= 4096 ? 2 : 4);
  const dim3 grid((unsigned)blocks);
#define OZK_PAIR(W, V, G, N) \
  hipLaunchKernelGGL((deconstruct_pair_kernel<W, V, G, N>), grid, dim3(256), 0, s, p)
#define OZK_PAIR_G(W, V, N)              \
  if (g == 1) OZK_PAIR(W, V, 1, N);      \
  else if (g == 2) OZK_PAIR(W, V, 2, N); \
  else OZK_PAIR(W, V, 4, N)
#define OZK_PAIR_N(W, V)                        \
  if (norm) { OZK_PAIR_G(W, V, true); }         \
  else { OZK_PAIR_G(W, V, false); }
  if (ka.wide && vec) { OZK_PAIR_N(true, true) }
  else if (ka.wide) { OZK_PAIR_N(true, false) }
  else if (vec) { OZK_PAIR_N(false, true) }
  else { OZK_PAIR_N(false, false) }
#undef OZK_PAIR_N
#undef OZK_PAIR_G
#undef OZK_PAIR
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

int64_t norm_chunks(int64_t rows, int64_t cols, int axis) {
  return axis == 0 ? (cols + 2047) / 2048 : (rows + 127) / 128;
}

int launch_norm_exps(const double* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                     int alpha, uint64_t* pmax, double* ps, int32_t* exps, hipStream_t s) {
  const int64_t lines = axis == 0 ? rows : cols;
  if (lines <= 0) return OZK_OK;
  const int64_t chunks = norm_chunks(rows, cols, axis);
  if (chunks > 0) {
    if (axis == 0) {
      if (rows > 65535) return OZK_EUNSUPPORTED;
      hipLaunchKernelGGL(norm_partials_rows_kernel, dim3((unsigned)chunks, (unsigned)rows),
                         dim3(256), 0, s, x, cols, ldx, pmax, ps);
    } else {
      hipLaunchKernelGGL(norm_partials_cols_kernel,
                         dim3((unsigned)((cols + 255) / 256), (unsigned)chunks), dim3(256), 0, s,
                         x, rows, cols, ldx, pmax, ps);
    }
    if (hipGetLastError() != hipSuccess) return OZK_EHIP;
  }
  const int64_t sl = axis == 0 ? chunks : 1, sc = axis == 0 ? 1 : cols;
  hipLaunchKernelGGL(exps_norm_kernel, dim3((unsigned)((lines + 15) / 16)), dim3(256), 0, s,
                     pmax, ps, lines, chunks, sl, sc, alpha, exps);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

int launch_line_exps(const double* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                     int p_bits, uint64_t* maxbits, int32_t* exps, hipStream_t s) {
  const int64_t lines = axis == 0 ? rows : cols;
  if (lines <= 0) return OZK_OK;
  int st;
  if ((st = launch_fill_u64(maxbits, lines, 0, s)) != OZK_OK) return st;
  if ((st = launch_absmax(x, rows, cols, ldx, axis, maxbits, s)) != OZK_OK) return st;
  hipLaunchKernelGGL(exps_from_maxbits_kernel, dim3((unsigned)((lines + 255) / 256)), dim3(256), 0,
                     s, maxbits, lines, p_bits, exps);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

int launch_residues_rows_fused(const double* x, int64_t rows, int64_t cols, int64_t ldx, int r,
                               int scaling, int width, int8_t* planes, int64_t ldp,
                               int64_t plane_stride, int32_t* exps, hipStream_t s) {
  if (rows <= 0) return OZK_OK;
  if (!residue_consts(r, width)) return OZK_EINVAL;
  const ResidueConsts& K = *residue_consts(r, width);
  const bool wide = K.wide != 0;
  const int norm = scaling == OZK_SCALING_NORM;
#define OZK_FUSED(NT, G)                                                                      \
  return wide ? launch_fused<true, NT, G>(x, rows, cols, ldx, K, norm, width, planes, ldp,    \
                                          plane_stride, exps, s)                              \
              : launch_fused<false, NT, G>(x, rows, cols, ldx, K, norm, width, planes, ldp,   \
                                           plane_stride, exps, s)
  if (cols <= 2048) { OZK_FUSED(256, 1); }
  if (cols <= 4096) { OZK_FUSED(256, 2); }
  if (cols <= 8192) { OZK_FUSED(256, 4); }
  if (cols <= 16384) { OZK_FUSED(512, 4); }
  OZK_FUSED(1024, 4);
#undef OZK_FUSED
}

}  // namespace ozk
