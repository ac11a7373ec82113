// CRT reconstruction and inverse scaling: the per-output reconstruction term of Ozaki
// scheme II ([TME4] abstract).  Each thread reconstructs 4 consecutive outputs of a row.
//
// Given symmetric residues c_l (|c_l| <= 128) of the exact integer X modulo m_l:
//   1. q = round(sum_l c_l * RN(E_l / M)).  The exact value of the sum is q + X/M with
//      |X| <= 2^Q <= (M-1)/2, and 1/2 - 2^Q/M >= 0.0142 for every r <= 20, far above
//      the < 2^-30 error of the fp64 sum, so q is exact.
//   2. X = sum_l c_l E_l - q M, in 2^40 limbs held in fp64: every limb sum stays below
//      2^53 (at most 20 * 2^47 + 2^51.4), so all fp64 operations are exact.
//   3. Limbs are normalised to digits in [0, 2^40) and the sign split off; RN(|X| 2^-s)
//      is formed with one fp64 rounding of the top digits plus an exact tie correction
//      (round_digits), or, for a subnormal result, by integer rounding at the reduced
//      precision, so the output is rounded exactly once.
// The constants come from the compile-time table in __constant__ memory; each block
// stages the r(L+1)+L values it needs in LDS (compile-time r), and every constant is
// read once per 4 outputs, so none of them has to live in scalar registers.
#include "ozk_internal.h"
#include "rns_table.h"

namespace ozk {

__constant__ RnsTable d_rns = make_rns_table();

namespace {

__device__ __forceinline__ uint64_t u64_of(double d) {  // d integer in [0, 2^53)
  const double hi = __builtin_floor(d * 0x1p-32);
  const double lo = __builtin_fma(-hi, 0x1p32, d);
  return ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo;
}

// RN(mag * 2^-s) for mag = w2:w1:w0 (little-endian 64-bit words), mag != 0.
__device__ __forceinline__ double round_scaled_words(uint64_t w0, uint64_t w1, uint64_t w2,
                                                     int s) {
  uint64_t top;
  bool sticky;
  int lead;  // bit index of the leading 1 of mag
  if (w2) {
    const int sh = __builtin_clzll(w2);
    top = sh ? (w2 << sh) | (w1 >> (64 - sh)) : w2;
    sticky = (sh ? (w1 << sh) : w1) != 0 || w0 != 0;
    lead = 191 - sh;
  } else if (w1) {
    const int sh = __builtin_clzll(w1);
    top = sh ? (w1 << sh) | (w0 >> (64 - sh)) : w1;
    sticky = (sh ? (w0 << sh) : w0) != 0;
    lead = 127 - sh;
  } else {
    const int sh = __builtin_clzll(w0);
    top = w0 << sh;
    sticky = false;
    lead = 63 - sh;
  }
  const int E = lead - s;  // mag * 2^-s lies in [2^E, 2^(E+1))
  if (E > 1023) return __builtin_huge_val();
  const int keep = E >= -1022 ? 53 : E + 1075;  // significant bits the result holds
  if (keep < 0) return 0.0;
  uint64_t mant;
  bool up;
  if (keep == 0) {
    mant = 0;
    up = top > 0x8000000000000000ull || (top == 0x8000000000000000ull && sticky);
  } else {
    const int drop = 64 - keep;
    mant = top >> drop;
    const uint64_t rem = top & ((1ull << drop) - 1);
    const uint64_t half = 1ull << (drop - 1);
    up = rem > half || (rem == half && (sticky || (mant & 1)));
  }
  mant += up ? 1 : 0;
  // mant <= 2^53: the conversion is exact; ldexp scales exactly (or overflows to Inf).
  return __builtin_ldexp((double)mant, E >= -1022 ? E - 52 : -1074);
}

// RN(V * 2^-s) for V = sum_p d[p] 2^(40 p), digits d[p] integers in [0, 2^40).
// Fast path, all in exact fp64 arithmetic: take the top nonzero digit H and the digits
// below it so that S = H*2^40 + next (or (H*2^40 + next)*2^40 + next2 when H < 2^13) has
// at least 54 bits; fma rounds S once (RNE), and its error err = S - RN(S) is exact.
// Digits further down add a fraction 0 <= eps < 1 (in units of S); S is an integer and
// every rounding midpoint at >= 54 bits is an integer, so eps can only matter when S sits
// exactly on a midpoint below it (err = +ulp/2): then the true value lies above the
// midpoint and RN rounds up.  Scaling by 2^(base - s) is exact for a normal result; a
// subnormal (or zero) result takes the integer path below.
template <int L>
__device__ __forceinline__ double round_digits(const double (&d)[4], int s) {
  double h, lo, lo2;
  bool rest;  // any nonzero digit below lo2
  int top;
  if (L > 3 && d[3] != 0.0) {
    top = 3; h = d[3]; lo = d[2]; lo2 = d[1]; rest = d[0] != 0.0;
  } else if (d[2] != 0.0) {
    top = 2; h = d[2]; lo = d[1]; lo2 = d[0]; rest = false;
  } else if (d[1] != 0.0) {
    top = 1; h = d[1]; lo = d[0]; lo2 = 0.0; rest = false;
  } else {
    top = 0; h = d[0]; lo = 0.0; lo2 = 0.0; rest = false;
  }
  if (h == 0.0) return 0.0;
  double S, err;
  bool below;  // nonzero digits below the ones folded into S
  int base;
  if (h >= 8192.0) {  // H has >= 14 bits: H*2^40 + lo has >= 54
    S = __builtin_fma(h, 0x1p40, lo);
    err = __builtin_fma(h, 0x1p40, -S) + lo;
    below = lo2 != 0.0 || rest;
    base = 40 * (top - 1);
  } else {
    const double t = __builtin_fma(h, 0x1p40, lo);  // < 2^53: exact
    S = __builtin_fma(t, 0x1p40, lo2);
    err = __builtin_fma(t, 0x1p40, -S) + lo2;
    below = rest;
    base = 40 * (top - 2);
  }
  const int e = __builtin_amdgcn_frexp_exp(S) - 1;  // ilogb(S)
  const double half_ulp = __builtin_ldexp(1.0, e - 53);
  if (below && err == half_ulp) S += 2.0 * half_ulp;
  const int E = e + base - s;  // exponent of the result (before a possible carry)
  if (E >= -1021) return __builtin_ldexp(S, base - s);
  // Subnormal or underflowing result: exact integer rounding at the reduced precision.
  const uint64_t d0 = u64_of(d[0]), d1 = u64_of(d[1]), d2 = u64_of(d[2]);
  const uint64_t d3 = L > 3 ? u64_of(d[3]) : 0;
  const uint64_t w0 = d0 | (d1 << 40);
  const uint64_t w1 = (d1 >> 24) | (d2 << 16) | (d3 << 56);
  const uint64_t w2 = d3 >> 8;
  return round_scaled_words(w0, w1, w2, s);
}

// Exact integer X of 4 outputs from their residues and the RNS constants in LDS,
// rounded to fp64 with the shift s[u].
template <int R>
__device__ __forceinline__ void reconstruct4(const int32_t (&word)[R], const double* __restrict__ sc,
                                             const int (&s)[4], const bool (&nan)[4],
                                             double (&out)[4]) {
  constexpr int L = R <= 15 ? 3 : 4;
  // sc layout: frac[R], e[R][L], m[L]
  double qf[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int l = 0; l < R; ++l) {
    const double fr = sc[l];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      qf[u] = __builtin_fma((double)(int)(int8_t)(word[l] >> (8 * u)), fr, qf[u]);
  }
  double x[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const double q = __builtin_rint(qf[u]);
#pragma unroll
    for (int p = 0; p < L; ++p) x[u][p] = -q * sc[R + R * L + p];  // |q| < 2^11.4: exact
#pragma unroll
    for (int p = L; p < 4; ++p) x[u][p] = 0.0;
  }
#pragma unroll
  for (int l = 0; l < R; ++l) {
    double cd[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) cd[u] = (double)(int)(int8_t)(word[l] >> (8 * u));
#pragma unroll
    for (int p = 0; p < L; ++p) {
      const double e = sc[R + l * L + p];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u][p] = __builtin_fma(cd[u], e, x[u][p]);
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    double* xu = x[u];
#pragma unroll
    for (int p = 0; p < L - 1; ++p) {  // digits 0..L-2 in [0, 2^40); sign in digit L-1
      const double carry = __builtin_floor(xu[p] * 0x1p-40);
      xu[p] = __builtin_fma(-carry, 0x1p40, xu[p]);
      xu[p + 1] += carry;
    }
    const bool neg = xu[L - 1] < 0.0;
    if (neg) {
#pragma unroll
      for (int p = 0; p < L; ++p) xu[p] = -xu[p];
#pragma unroll
      for (int p = 0; p < L - 1; ++p) {
        const double carry = __builtin_floor(xu[p] * 0x1p-40);
        xu[p] = __builtin_fma(-carry, 0x1p40, xu[p]);
        xu[p + 1] += carry;
      }
    }
    double o = round_digits<L>(x[u], s[u]);
    o = neg ? -o : o;
    out[u] = nan[u] ? __builtin_nan("") : o;
  }
}

template <typename T>
__device__ __forceinline__ int symmetric(T v, int l, int mod) {
  if (sizeof(T) == 1) return (int)v;
  // raw int32 products: reduce to the symmetric residue first
  if (mod == 256) return (int)(int8_t)(v & 0xff);
  constexpr double kMagicD = 6755399441055744.0;
  const double d = (double)v;
  const double q = __builtin_fma(d, d_rns.inv[l], kMagicD) - kMagicD;
  return (int)__builtin_fma(-q, (double)mod, d);
}

template <int R, typename T>
__global__ __launch_bounds__(256) void crt_kernel(int64_t m, int64_t n, const T* __restrict__ res,
                                                  int64_t ldr, int64_t stride_r,
                                                  const int32_t* __restrict__ ea,
                                                  const int32_t* __restrict__ eb,
                                                  double* __restrict__ c, int64_t ldc) {
  constexpr int L = R <= 15 ? 3 : 4;
  constexpr int kConsts = R + R * L + L;
  __shared__ double sc[kConsts];
  for (int t = threadIdx.x; t < kConsts; t += blockDim.x) {
    double v;
    if (t < R)
      v = d_rns.frac[R][t];
    else if (t < R + R * L)
      v = d_rns.e_limb[R][(t - R) / L][(t - R) % L];
    else
      v = d_rns.m_limb[R][t - R - R * L];
    sc[t] = v;
  }
  __syncthreads();
  // Flat index over (row, quad of 4 columns).
  const int64_t nq = (n + 3) / 4;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= m * nq) return;
  const int64_t i = g / nq;
  const int64_t j0 = (g - i * nq) * 4;
  const int cnt = n - j0 >= 4 ? 4 : (int)(n - j0);
  int f[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) f[u] = u < cnt ? eb[j0 + u] : 0;
  const bool vec = cnt == 4 && sizeof(T) == 1 && ((ldr | stride_r | j0) & 3) == 0;
  {
    const int32_t e_i = ea[i];
    const T* src = res + i * ldr + j0;
    // Symmetric residues of the 4 outputs, one byte each, packed per modulus.
    int32_t word[R];
    if (vec) {
#pragma unroll
      for (int l = 0; l < R; ++l) word[l] = *reinterpret_cast<const int32_t*>(src + l * stride_r);
    } else {
#pragma unroll
      for (int l = 0; l < R; ++l) {
        uint32_t w = 0;
        for (int u = 0; u < cnt; ++u)
          w |= ((uint32_t)symmetric<T>(src[l * stride_r + u], l, d_rns.moduli[l]) & 0xffu)
               << (8 * u);
        word[l] = (int32_t)w;
      }
    }
    int s[4];
    bool nan[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      s[u] = e_i + f[u];
      nan[u] = e_i == INT32_MIN || f[u] == INT32_MIN;
    }
    double out[4];
    reconstruct4<R>(word, sc, s, nan, out);
    double* dst = c + i * ldc + j0;
    if (cnt == 4 && ((ldc | j0) & 1) == 0) {
      *reinterpret_cast<double2*>(dst) = make_double2(out[0], out[1]);
      *reinterpret_cast<double2*>(dst + 2) = make_double2(out[2], out[3]);
    } else {
      for (int u = 0; u < cnt; ++u) dst[u] = out[u];
    }
  }
}

template <int R>
void launch_r(dim3 grid, hipStream_t s, int64_t m, int64_t n, const void* res, int is_i32,
              int64_t ldr, int64_t stride_r, const int32_t* ea, const int32_t* eb, double* c,
              int64_t ldc) {
  if (is_i32)
    hipLaunchKernelGGL((crt_kernel<R, int32_t>), grid, dim3(256), 0, s, m, n,
                       (const int32_t*)res, ldr, stride_r, ea, eb, c, ldc);
  else
    hipLaunchKernelGGL((crt_kernel<R, int8_t>), grid, dim3(256), 0, s, m, n, (const int8_t*)res,
                       ldr, stride_r, ea, eb, c, ldc);
}

template <int... Rs>
struct Dispatch;

template <>
struct Dispatch<> {
  static void go(int, dim3, hipStream_t, int64_t, int64_t, const void*, int, int64_t, int64_t,
                 const int32_t*, const int32_t*, double*, int64_t) {}
};

template <int R0, int... Rs>
struct Dispatch<R0, Rs...> {
  static void go(int r, dim3 g, hipStream_t s, int64_t m, int64_t n, const void* res, int i32,
                 int64_t ldr, int64_t sr, const int32_t* ea, const int32_t* eb, double* c,
                 int64_t ldc) {
    if (r == R0)
      launch_r<R0>(g, s, m, n, res, i32, ldr, sr, ea, eb, c, ldc);
    else
      Dispatch<Rs...>::go(r, g, s, m, n, res, i32, ldr, sr, ea, eb, c, ldc);
  }
};

}  // namespace

int launch_crt(int64_t m, int64_t n, int r, const void* res, int res_is_i32, int64_t ldr,
               int64_t stride_r, const int32_t* ea, const int32_t* eb, double* c, int64_t ldc,
               hipStream_t s) {
  if (m <= 0 || n <= 0) return OZK_OK;
  if (r < 1 || r > kMaxModuli) return OZK_EINVAL;
  const int64_t blocks = (m * ((n + 3) / 4) + 255) / 256;
  if (blocks > 0x7fffffff) return OZK_EUNSUPPORTED;
  dim3 grid((unsigned)blocks);
  Dispatch<1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20>::go(
      r, grid, s, m, n, res, res_is_i32, ldr, stride_r, ea, eb, c, ldc);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

}  // namespace ozk
