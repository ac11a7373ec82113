// On-the-fly emulated GEMV / low-batch GEMV through base-256 digits of the scaled
// integers: the memory-bound case of [TME4] abstract with the per-element deconstruction
// cut to one fp64 FMA and two integer XORs.
//
// The residue products Y_l = A_l X_l (mod m_l) only need each scaled integer a' =
// RNE(a 2^e) modulo m_l.  Writing a' in signed base-256 digits, a' = sum_j d_j 256^j,
// gives a' = sum_j d_j w_jl (mod m_l) with w_jl = 256^j mod m_l, so
//
//   sum_h a'_ih x_hl  =  sum_h sum_j d_ihj (w_jl x_hl mod m_l)     (mod m_l),
//
// an exact int8 x int8 product over K' = 8 k digit positions against "weighted digit
// planes" X'_l[h, j] = smod(w_jl x_hl, m_l) computed once per call from the residues of
// X.  The digits come straight out of the fp64 bit pattern: with the constant
// C = 2^52 + K, K = 0x8808080808080,
//
//   t = RN(a 2^e + C) = C + RNE(a 2^e)            (|a'| <= 2^50: ulp(t) = 1, C even)
//
// holds u = K + a' in its 52 mantissa bits, and since K has bytes 0x80 in positions
// 0..5 and 8 in the nibble above them,
//
//   a' = sum_{j<6} (b_j - 128) 256^j + (b_6 - 56) 2^48,
//
// where b_j are the bytes of t (b_6 = 0x30 + that nibble lies in [52, 60]).  XORing bytes
// 0..5 with 0x80 turns them into the int8 values b_j - 128; byte 6 is fed as is and the
// constant -56 w_6l sum_h x_hl (mod m_l) is added once per output column; byte 7 (the
// exponent) meets a zero weight.  The MFMA therefore reads the eight bytes of t directly.
//
// int32 accumulation stays exact over slices of at most kSliceElems = 8192 elements
// (|digit| <= 128, |weight| <= 128, 7 weighted digits per element: < 2^30); longer K is
// split over the grid's y dimension and the slices' residues are summed in a last pass.
#include <type_traits>

#include "ozk_internal.h"

namespace ozk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kSliceElems = 8192;          // elements of K per int32 accumulation
constexpr int kSuper = 16;                 // elements per super-chunk (128 digit bytes)
constexpr int kRowsPerBlock = 128;         // 4 waves x 2 row tiles of 16
constexpr int kMaxTiles = 16;              // 16-column MFMA tiles per pass (r * nrhs <= 256)

struct DigitModuli {
  int32_t m[kMaxModuli];
  double inv[kMaxModuli];
  int32_t w[kMaxModuli][8];   // smod(256^j mod m, m), j = 0..6; w[.][7] = 0
};

constexpr int smod_c(int64_t x, int64_t m) {
  int64_t r = x % m;
  if (r < 0) r += m;
  // symmetric: [-floor(m/2), ceil(m/2) - 1]
  if (r >= (m + 1) / 2) r -= m;
  return (int)r;
}

constexpr DigitModuli make_digit_moduli() {
  DigitModuli d{};
  const int32_t mods[kMaxModuli] = {256, 255, 253, 251, 247, 241, 239, 233, 229, 227,
                                    223, 217, 211, 199, 197, 193, 191, 181, 179, 173};
  for (int l = 0; l < kMaxModuli; ++l) {
    d.m[l] = mods[l];
    d.inv[l] = 1.0 / (double)mods[l];
    int64_t p = 1;
    for (int j = 0; j < 7; ++j) {
      d.w[l][j] = smod_c(p, mods[l]);
      p = (p * 256) % mods[l];
    }
    d.w[l][7] = 0;
  }
  return d;
}

__constant__ DigitModuli d_dm = make_digit_moduli();

// Symmetric residue of an int32 modulo m_l (odd m: exact rounded quotient through fp64,
// never a tie; m = 256: the low byte).
__device__ __forceinline__ int sym_mod(int v, int m, double inv) {
  if (m == 256) return (int)(int8_t)(v & 0xff);
  constexpr double kMagicD = 6755399441055744.0;
  const double q = __builtin_fma((double)v, inv, kMagicD) - kMagicD;
  return (int)__builtin_fma(-q, (double)m, (double)v);
}

// Position of digit j of element h inside a column of the weighted digit planes, in the
// order the main kernel feeds the MFMA: super-chunk s = h / 16 holds 2 K steps of 64
// bytes; in K step ks, lane group g (lanes 16 g .. 16 g + 15) supplies elements
// 16 s + 4 g + 2 ks + {0, 1}.
__device__ __forceinline__ int64_t digit_pos(int64_t h) {
  const int64_t s = h >> 4;
  const int rem = (int)(h & 15);
  const int g = rem >> 2, ks = (rem >> 1) & 1, u = rem & 1;
  return s * 128 + ks * 64 + g * 16 + u * 8;
}

// ------------------------------------------------------------------ weighted X digits
// grid (ncols, ceil(kp / 2048)): block (n, chunk) writes xd[n][digit_pos(h) + j] =
// smod(w_jl x_h, m_l) for its 2048 elements h of column n = l * nrhs + c and the partial
// sum of x_h over them to psum[n][chunk] (the combine pass turns the sums into the
// byte-6 correction).
constexpr int kPrepElems = 2048;

__global__ __launch_bounds__(256) void xdigits_kernel(const int8_t* __restrict__ xp,
                                                      int64_t kp, int64_t x_stride, int nrhs,
                                                      int8_t* __restrict__ xd,
                                                      int32_t* __restrict__ psum) {
  const int n = blockIdx.x;
  const int l = n / nrhs, c = n - l * nrhs;
  const int m = d_dm.m[l];
  const double inv = d_dm.inv[l];
  const int8_t* x = xp + (int64_t)l * x_stride + (int64_t)c * kp;
  int8_t* out = xd + (int64_t)n * 8 * kp;
  int w[7];
#pragma unroll
  for (int j = 0; j < 7; ++j) w[j] = d_dm.w[l][j];
  int sum = 0;
  const int64_t h0 = (int64_t)blockIdx.y * kPrepElems;
  for (int64_t h = h0 + threadIdx.x; h < kp && h < h0 + kPrepElems; h += 256) {
    const int xv = x[h];
    sum += xv;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) lo |= ((uint32_t)sym_mod(w[j] * xv, m, inv) & 0xffu) << (8 * j);
#pragma unroll
    for (int j = 4; j < 7; ++j)
      hi |= ((uint32_t)sym_mod(w[j] * xv, m, inv) & 0xffu) << (8 * (j - 4));
    *reinterpret_cast<uint2*>(out + digit_pos(h)) = make_uint2(lo, hi);
  }
  // Wave sums through cross-lane adds, then the four waves through LDS.
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  __shared__ int wsum[4];
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = sum;
  __syncthreads();
  if (threadIdx.x == 0)
    psum[(int64_t)n * gridDim.y + blockIdx.y] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

// ------------------------------------------------------------------ main kernel
// grid (ceil(m / 128), slices, passes); 4 waves, each 2 row tiles of 16 rows of A against
// NT tiles of 16 output columns (columns n0 .. n0 + 16 NT - 1, n0 = 256 blockIdx.z) on
// v_mfma_i32_16x16x64_i8, over the K slice blockIdx.y.  The block stages the 128 digit
// bytes per column of G super-chunks (16 elements each) at a time in LDS,
// double-buffered, one barrier per group; the 16-byte chunk index is XOR-swizzled by
// (column >> 1) & 7 so that the 16 lanes of a fragment read hit distinct banks.  Lane
// (row lane % 16, group g = lane / 16) turns the 4 fp64 of its row it holds per
// super-chunk (elements 4 g .. 4 g + 3) into the MFMA operands of the super-chunk's two K
// steps, for each of its two row tiles; the two K steps of an output tile go to the
// matrix core back to back.  A is prefetched two super-chunks ahead, and the X' loads of
// the next group are issued at the start of a group and written to LDS at its end.
// G super-chunks per LDS stage, measured at 32768^2, r = 14 (ms for G = 1 / 2): 2 columns
// (NT = 2) 1.50 / 1.56, 4 columns (NT = 4) 1.86-1.90 / 1.53, 6 columns (NT = 6) 1.77 /
// 1.64-1.68, 8 columns (NT = 7) 1.80-1.84 / 1.82-1.87.  Three or four row tiles per wave
// (fewer X' reads per MFMA) were slower at every column count: the accumulators leave
// room for one wave per SIMD only.
template <int NT>
constexpr int digits_stage_group() {
  return NT >= 3 && NT <= 6 ? 2 : 1;
}

template <int NT, int G>
struct DigitsShape {
  static constexpr int kStageBytes = G * NT * 16 * 128;
  static constexpr int kChunks = kStageBytes / 16;
  static constexpr int kLoads = (kChunks + 255) / 256;      // 16-byte loads per thread
};

template <int NT, int G, bool kFast>
__global__ __launch_bounds__(256) void gemv_digits_kernel(
    const double* __restrict__ a, int64_t m, int64_t k, int64_t lda,
    const int32_t* __restrict__ exps, const int8_t* __restrict__ xd, int64_t kp, int nrhs,
    int ncols, int8_t* __restrict__ part, int vec) {
  using S = DigitsShape<NT, G>;
  __shared__ __attribute__((aligned(16))) int8_t xs[2][S::kStageBytes];
  constexpr double kDigitMagic = 0x1.8808080808080p+52;   // 2^52 + 0x8808080808080
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int grp = lane >> 4;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (tid >> 6)) * 32;
  int64_t rows[2];
  rows[0] = row0 + (lane & 15);
  rows[1] = rows[0] + 16;
  const int slice = blockIdx.y;
  const int n0 = blockIdx.z * kMaxTiles * 16;
  const int64_t h_begin = (int64_t)slice * kSliceElems;
  const int64_t h_end = h_begin + kSliceElems < kp ? h_begin + kSliceElems : kp;
  const int64_t nsc = (h_end - h_begin) / kSuper;

  // Per row tile: 2^e as two normal factors (s0 = 1 unless the row is so small that
  // e > 1023).  A row holding Inf/NaN (exponent INT32_MIN) contributes residues 0 on the
  // general path; the fast path below feeds it as it is: its residues are then
  // meaningless, and the reconstruction turns every output of the row into NaN either way.
  double s0[2], s1[2];
  int64_t klim[2];
  const double* pa[2];
  bool tiny_any = false;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int64_t row = rows[rt] < m ? rows[rt] : m - 1;
    int e = exps[row];
    const bool bad = e == INT32_MIN;
    if (bad) e = 0;
    klim[rt] = bad ? 0 : k;
    s1[rt] = __builtin_ldexp(1.0, e < 1023 ? e : 1023);
    s0[rt] = __builtin_ldexp(1.0, e < 1023 ? 0 : e - 1023);
    tiny_any |= e > 1023;
    pa[rt] = a + row * lda;
  }
  const bool tiny = __ballot(tiny_any) != 0;   // wave-uniform

  v4i acc[2][NT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[rt][q][v] = 0;

  // Staging of group g: load i of a thread is chunk c = 256 i + tid of the stage, i.e.
  // chunk c % 8 of column (c / 8) % (16 NT) in super-chunk G g + c / (128 NT).  Columns
  // past ncols are not loaded (their MFMA results are never stored).
  auto x_load = [&](v4i (&xr)[S::kLoads], int64_t g) {
#pragma unroll
    for (int i = 0; i < S::kLoads; ++i) {
      const int c = 256 * i + tid;
      const int64_t sc = g * G + c / (128 * NT);
      const int col = (c >> 3) % (16 * NT);
      const int n = n0 + col;
      if (c < S::kChunks && n < ncols && sc < nsc)
        xr[i] = *reinterpret_cast<const v4i*>(xd + (int64_t)n * 8 * kp +
                                              (h_begin / kSuper + sc) * 128 + (c & 7) * 16);
    }
  };
  auto x_store = [&](const v4i (&xr)[S::kLoads], int buf) {
#pragma unroll
    for (int i = 0; i < S::kLoads; ++i) {
      const int c = 256 * i + tid;
      if (c < S::kChunks) {
        const int w = c / (128 * NT);
        const int col = (c >> 3) % (16 * NT), ch = c & 7;
        *reinterpret_cast<v4i*>(&xs[buf][w * (NT * 2048) + col * 128 +
                                         ((ch ^ ((col >> 1) & 7)) << 4)]) = xr[i];
      }
    }
  };
  // The 4 fp64 of each row tile this lane feeds in super-chunk sc (elements
  // 16 sc + 4 grp .. + 3).
  auto load_a = [&](double (&v)[2][4], int64_t sc) {
    const int64_t h0 = h_begin + sc * kSuper + 4 * grp;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      if (vec && h0 + 4 <= klim[rt]) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const double2 d = *reinterpret_cast<const double2*>(pa[rt] + h0 + 2 * u);
          v[rt][2 * u] = d.x;
          v[rt][2 * u + 1] = d.y;
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[rt][u] = h0 + u < klim[rt] ? pa[rt][h0 + u] : 0.0;
      }
    }
  };

  // Fast path (chosen by the host: rows 16-byte aligned, k a multiple of 16, so every
  // super-chunk below k is whole): every global load of the loop is issued without a
  // condition, from addresses clamped into A and X' (super-chunks past k feed zeros), in
  // one fixed order per super-chunk (staging loads, then A two super-chunks ahead, then
  // the MFMAs), so the compiler's waits count exactly the loads a super-chunk needs and
  // leave A's loads in flight (32768^2, r = 14, 8 columns: 1.835 -> 1.790 ms).
  int64_t nsc_k = (k - h_begin) / kSuper;
  nsc_k = nsc_k < nsc ? nsc_k : nsc;
  auto load_a_fast = [&](double (&v)[2][4], int64_t sc) {
    const int64_t h0 = (sc < nsc_k ? sc : nsc_k - 1) * kSuper + h_begin + 4 * grp;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const double2 d = *reinterpret_cast<const double2*>(pa[rt] + h0 + 2 * u);
        v[rt][2 * u] = d.x;
        v[rt][2 * u + 1] = d.y;
      }
  };
  // A lane past the stage's last chunk loads and stores that chunk again (the same bytes
  // to the same place), a column past ncols reads the last live column.
  uint32_t x_src[S::kLoads], x_dst[S::kLoads];
#pragma unroll
  for (int i = 0; i < S::kLoads; ++i) {
    int c = 256 * i + tid;
    c = c < S::kChunks ? c : S::kChunks - 1;
    const int w = c / (128 * NT);
    const int col = (c >> 3) % (16 * NT), ch = c & 7;
    const int n = n0 + col < ncols ? n0 + col : ncols - 1;
    x_src[i] = (uint32_t)((int64_t)n * 8 * kp + (h_begin / kSuper + w) * 128 + ch * 16);
    x_dst[i] = (uint32_t)(w * (NT * 2048) + col * 128 + ((ch ^ ((col >> 1) & 7)) << 4));
  }
  auto x_load_fast = [&](v4i (&xr)[S::kLoads], int64_t g) {
    const int8_t* base = xd + g * G * 128;
#pragma unroll
    for (int i = 0; i < S::kLoads; ++i) xr[i] = *reinterpret_cast<const v4i*>(base + x_src[i]);
  };
  auto x_store_fast = [&](const v4i (&xr)[S::kLoads], int buf) {
#pragma unroll
    for (int i = 0; i < S::kLoads; ++i) *reinterpret_cast<v4i*>(&xs[buf][x_dst[i]]) = xr[i];
  };

  v4i xr[S::kLoads];
  const int64_t ngroups = (nsc + G - 1) / G;
  // One super-chunk: MFMAs on v (then v is reloaded with super-chunk sc + 2).
  auto step = [&](double (&v)[2][4], int64_t sc, auto tiny_tag, auto within_tag) {
    constexpr bool kTiny = decltype(tiny_tag)::value;
    constexpr int within = decltype(within_tag)::value;   // sc % G
    const int64_t g = sc / G;
    const int buf = (int)(g & 1);
    const bool more = g + 1 < ngroups;
    if (kFast) {
      if (within == 0) x_load_fast(xr, more ? g + 1 : g);
      __builtin_amdgcn_sched_barrier(0);   // the staging loads go out first
    } else if (within == 0 && more) {
      x_load(xr, g + 1);
    }
    const int8_t* xb = &xs[buf][within * (NT * 2048)];
    v4i frag[2][2];
    const bool past_k = kFast && sc >= nsc_k;   // wave-uniform
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        double x0 = past_k ? 0.0 : v[rt][2 * ks], x1 = past_k ? 0.0 : v[rt][2 * ks + 1];
        if (kTiny) {
          x0 *= s0[rt];
          x1 *= s0[rt];
        }
        const uint64_t t0 =
            (uint64_t)__double_as_longlong(__builtin_fma(x0, s1[rt], kDigitMagic));
        const uint64_t t1 =
            (uint64_t)__double_as_longlong(__builtin_fma(x1, s1[rt], kDigitMagic));
        frag[rt][ks][0] = (int)((uint32_t)t0 ^ 0x80808080u);
        frag[rt][ks][1] = (int)((uint32_t)(t0 >> 32) ^ 0x00008080u);
        frag[rt][ks][2] = (int)((uint32_t)t1 ^ 0x80808080u);
        frag[rt][ks][3] = (int)((uint32_t)(t1 >> 32) ^ 0x00008080u);
      }
    if (kFast) {
      load_a_fast(v, sc + 2);
      __builtin_amdgcn_sched_barrier(0);   // then A two super-chunks ahead, then the MFMAs
    } else if (sc + 2 < nsc) {
      load_a(v, sc + 2);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = nt * 16 + (lane & 15);
      const v4i xf0 =
          *reinterpret_cast<const v4i*>(xb + col * 128 + (((0 + grp) ^ ((col >> 1) & 7)) << 4));
      const v4i xf1 =
          *reinterpret_cast<const v4i*>(xb + col * 128 + (((4 + grp) ^ ((col >> 1) & 7)) << 4));
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        acc[rt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(frag[rt][0], xf0, acc[rt][nt], 0, 0, 0);
        acc[rt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(frag[rt][1], xf1, acc[rt][nt], 0, 0, 0);
      }
    }
    if (kFast) {
      // the next group's stage (a harmless rewrite of the other buffer after the last)
      __builtin_amdgcn_sched_barrier(0);
      if (within == G - 1) {
        x_store_fast(xr, buf ^ 1);
        __syncthreads();
      }
    } else if (within == G - 1 || sc == nsc - 1) {
      if (more) x_store(xr, buf ^ 1);
      __syncthreads();
    }
  };
  auto run = [&](auto tiny_tag) {
    double va[2][4], vb[2][4];
    if (kFast) {
      load_a_fast(va, 0);
      load_a_fast(vb, 1);
      x_load_fast(xr, 0);
    } else {
      load_a(va, 0);
      if (nsc > 1) load_a(vb, 1);
      x_load(xr, 0);
    }
    x_store(xr, 0);
    __syncthreads();
    // nsc is a multiple of 4 (kp a multiple of 64), so the pair loop has no tail
    for (int64_t sc = 0; sc < nsc; sc += 2) {
      step(va, sc, tiny_tag, std::integral_constant<int, 0>{});
      step(vb, sc + 1, tiny_tag, std::integral_constant<int, 1 % G>{});
    }
  };
  if (tiny)
    run(std::true_type{});
  else
    run(std::false_type{});
  if (row0 >= m) return;

  // Residues of the slice: lane -> column n (one modulus per lane), register v -> row
  // 4 (lane / 16) + v of the row tile; four consecutive rows pack into one dword.
  int8_t* ps = part + (int64_t)slice * ncols * m;
  const bool vrows = (m & 3) == 0;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = n0 + nt * 16 + (lane & 15);
    if (n >= ncols) continue;
    const int l = n / nrhs;
    const int md = d_dm.m[l];
    const double inv = d_dm.inv[l];
    int8_t* pn = ps + (int64_t)n * m;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int64_t r0 = row0 + 16 * rt + 4 * grp;
      uint32_t w = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        w |= ((uint32_t)sym_mod(acc[rt][nt][u], md, inv) & 0xffu) << (8 * u);
      if (vrows && r0 + 4 <= m) {
        *reinterpret_cast<uint32_t*>(pn + r0) = w;
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (r0 + u < m) pn[r0 + u] = (int8_t)(w >> (8 * u));
      }
    }
  }
}

// ------------------------------------------------------------------ slice combine
// res[l][row][c] = smod(corr_n + sum_s part[s][n][row], m_l), n = l * nrhs + c, with the
// byte-6 correction corr_n = smod(-56 w_6l sum_h x_h, m_l) from the prep pass's sums.
__global__ __launch_bounds__(256) void digits_combine_kernel(
    const int8_t* __restrict__ part, int slices, int ncols, int64_t m, int nrhs,
    const int32_t* __restrict__ psum, int nchunks, int8_t* __restrict__ res) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)ncols * m) return;
  const int n = (int)(idx / m);
  const int64_t row = idx - (int64_t)n * m;
  const int l = n / nrhs, c = n - l * nrhs;
  const int md = d_dm.m[l];
  const double inv = d_dm.inv[l];
  int xs = 0;   // |sum_h x_h| <= 128 * 131072 < 2^31
  for (int q = 0; q < nchunks; ++q) xs += psum[(int64_t)n * nchunks + q];
  int v = sym_mod(-56 * d_dm.w[l][6] * sym_mod(xs, md, inv), md, inv);
  for (int s = 0; s < slices; ++s) v += part[((int64_t)s * ncols + n) * m + row];
  res[((int64_t)l * m + row) * nrhs + c] = (int8_t)sym_mod(v, md, inv);
}

template <int NT>
void launch_main(dim3 grid, hipStream_t s, const double* a, int64_t m, int64_t k, int64_t lda,
                 const int32_t* exps, const int8_t* xd, int64_t kp, int nrhs, int ncols,
                 int8_t* part, int vec) {
  constexpr int G = digits_stage_group<NT>();
  if (vec && k % kSuper == 0)
    hipLaunchKernelGGL((gemv_digits_kernel<NT, G, true>), grid, dim3(256), 0, s, a, m, k, lda,
                       exps, xd, kp, nrhs, ncols, part, vec);
  else
    hipLaunchKernelGGL((gemv_digits_kernel<NT, G, false>), grid, dim3(256), 0, s, a, m, k, lda,
                       exps, xd, kp, nrhs, ncols, part, vec);
}

}  // namespace

// Digits pay 8 MFMA K-bytes per element and output column; beyond 256 columns (16 tiles)
// the residue kernel, whose per-element cost does not grow with the columns, is faster.
bool gemv_digits_supported(int p_bits, int64_t ncols) { return p_bits <= 50 && ncols <= 256; }

size_t gemv_digits_workspace(int64_t m, int64_t kp, int r, int64_t nrhs, size_t* xd_bytes,
                             size_t* corr_bytes, size_t* part_bytes) {
  const int64_t ncols = (int64_t)r * nrhs;
  const int64_t slices = (kp + kSliceElems - 1) / kSliceElems;
  const int64_t chunks = (kp + kPrepElems - 1) / kPrepElems;
  *xd_bytes = (size_t)ncols * 8 * kp;
  *corr_bytes = (size_t)ncols * chunks * 4;
  *part_bytes = (size_t)slices * ncols * m;
  return *xd_bytes + *corr_bytes + *part_bytes;
}

int launch_gemv_digits(const double* a, int64_t m, int64_t k, int64_t lda, const int32_t* exps,
                       int r, const int8_t* xp, int64_t kp, int64_t x_stride, int nrhs,
                       int8_t* xd, int32_t* psum, int8_t* part, int8_t* res, hipStream_t s) {
  if (m <= 0) return OZK_OK;
  const int ncols = r * nrhs;
  const int chunks = (int)((kp + kPrepElems - 1) / kPrepElems);
  hipLaunchKernelGGL(xdigits_kernel, dim3((unsigned)ncols, (unsigned)chunks), dim3(256), 0, s,
                     xp, kp, x_stride, nrhs, xd, psum);
  if (hipGetLastError() != hipSuccess) return OZK_EHIP;
  const int slices = (int)((kp + kSliceElems - 1) / kSliceElems);
  const int tiles = (ncols + 15) / 16;
  const int passes = (tiles + kMaxTiles - 1) / kMaxTiles;
  const int nt = tiles < kMaxTiles ? tiles : kMaxTiles;
  const int vec = (reinterpret_cast<uintptr_t>(a) & 15) == 0 && (lda & 1) == 0;
  dim3 grid((unsigned)((m + kRowsPerBlock - 1) / kRowsPerBlock), (unsigned)slices,
            (unsigned)passes);
#define OZK_DIG(N)                                                                       \
  case N:                                                                                \
    launch_main<N>(grid, s, a, m, k, lda, exps, xd, kp, nrhs, ncols, part, vec);         \
    break
  switch (nt) {
    OZK_DIG(1); OZK_DIG(2); OZK_DIG(3); OZK_DIG(4); OZK_DIG(5); OZK_DIG(6); OZK_DIG(7);
    OZK_DIG(8); OZK_DIG(9); OZK_DIG(10); OZK_DIG(11); OZK_DIG(12); OZK_DIG(13); OZK_DIG(14);
    OZK_DIG(15); OZK_DIG(16);
    default: return OZK_EINVAL;
  }
#undef OZK_DIG
  if (hipGetLastError() != hipSuccess) return OZK_EHIP;
  const int64_t total = (int64_t)ncols * m;
  hipLaunchKernelGGL(digits_combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     s, part, slices, ncols, m, nrhs, psum, chunks, res);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

}  // namespace ozk
