// CRT reconstruction and inverse scaling: the per-output reconstruction term of Ozaki
// scheme II ([TME4] abstract).  One thread per output.
//
// Given symmetric residues c_l (|c_l| <= 128) of the exact integer X modulo m_l:
//   1. q = round(sum_l c_l * RN(E_l / M)).  The exact value of the sum is q + X/M with
//      |X| <= 2^Q <= (M-1)/2, and 1/2 - 2^Q/M >= 0.0142 for every r <= 20, far above
//      the < 2^-30 error of the fp64 sum, so q is exact.
//   2. X = sum_l c_l E_l - q M, in 2^40 limbs held in fp64: every limb sum stays below
//      2^53 (at most 20 * 2^47 + 2^51.4), so all fp64 operations are exact.
//   3. Limbs are normalised to digits in [0, 2^40), the sign split off, the magnitude
//      packed into three 64-bit words, and RN(|X| 2^-s) is formed by integer rounding
//      (half to even) at the precision of the result's binade: 53 bits for a normal
//      result, fewer for a subnormal one, so the output is rounded exactly once.
#include "ozk_internal.h"

namespace ozk {
namespace {

__device__ __forceinline__ int clz64(uint64_t x) { return __builtin_clzll(x); }

// RN(mag * 2^-s) for mag = w2:w1:w0 (little-endian 64-bit words), mag != 0.
__device__ double round_scaled_words(uint64_t w0, uint64_t w1, uint64_t w2, int s) {
  uint64_t top;
  bool sticky;
  int lead;  // bit index of the leading 1 of mag
  if (w2) {
    int sh = clz64(w2);
    top = sh ? (w2 << sh) | (w1 >> (64 - sh)) : w2;
    sticky = (sh ? (w1 << sh) : w1) != 0 || w0 != 0;
    lead = 191 - sh;
  } else if (w1) {
    int sh = clz64(w1);
    top = sh ? (w1 << sh) | (w0 >> (64 - sh)) : w1;
    sticky = (sh ? (w0 << sh) : w0) != 0;
    lead = 127 - sh;
  } else {
    int sh = clz64(w0);
    top = w0 << sh;
    sticky = false;
    lead = 63 - sh;
  }
  // Result exponent: mag * 2^-s lies in [2^E, 2^(E+1)).
  const int E = lead - s;
  if (E > 1023) return __builtin_huge_val();
  int keep = E >= -1022 ? 53 : E + 1075;  // significant bits the result can hold
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
  if (E >= -1022) return __builtin_ldexp((double)mant, E - 52);
  return __builtin_ldexp((double)mant, -1074);
}

template <typename T>
__global__ __launch_bounds__(256) void crt_kernel(int64_t m, int64_t n, const T* __restrict__ res,
                                                  int64_t ldr, int64_t stride_r,
                                                  const int32_t* __restrict__ ea,
                                                  const int32_t* __restrict__ eb,
                                                  double* __restrict__ c, int64_t ldc,
                                                  CrtConsts K) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  const int32_t f_j = eb[j];
  for (int64_t i = blockIdx.y; i < m; i += gridDim.y) {
  const int32_t e_i = ea[i];
  double* dst = c + i * ldc + j;
  if (e_i == INT32_MIN || f_j == INT32_MIN) {
    *dst = __builtin_nan("");
    continue;
  }
  constexpr double kMagicD = 6755399441055744.0;
  const int r = K.r;
  double cd[kMaxModuli];
  double qf = 0.0;
  const T* src = res + i * ldr + j;
#pragma unroll
  for (int l = 0; l < kMaxModuli; ++l) {
    if (l < r) {
      int v = (int)src[l * stride_r];
      if (sizeof(T) == 4) {  // raw products: reduce to the symmetric residue first
        const int mod = K.mod[l];
        if (mod == 256) {
          v = (int)(int8_t)(v & 0xff);
        } else {
          double d = (double)v;
          double q = __builtin_fma(d, K.inv[l], kMagicD) - kMagicD;
          v = (int)__builtin_fma(-q, (double)mod, d);
        }
      }
      cd[l] = (double)v;
      qf = __builtin_fma(cd[l], K.frac[l], qf);
    } else {
      cd[l] = 0.0;
    }
  }
  const double q = __builtin_rint(qf);
  double x[kMaxLimbs];
#pragma unroll
  for (int p = 0; p < kMaxLimbs; ++p) {
    double t = -q * K.m_limb[p];  // |q| < 2^11.4, limb < 2^40: exact
#pragma unroll
    for (int l = 0; l < kMaxModuli; ++l)
      if (l < r) t = __builtin_fma(cd[l], K.e_limb[l][p], t);
    x[p] = t;
  }
  // Normalise: digits 0..2 in [0, 2^40), the sign in digit 3.
#pragma unroll
  for (int p = 0; p < kMaxLimbs - 1; ++p) {
    double carry = __builtin_floor(x[p] * 0x1p-40);
    x[p] = __builtin_fma(-carry, 0x1p40, x[p]);
    x[p + 1] += carry;
  }
  const bool neg = x[kMaxLimbs - 1] < 0.0;
  if (neg) {
#pragma unroll
    for (int p = 0; p < kMaxLimbs; ++p) x[p] = -x[p];
#pragma unroll
    for (int p = 0; p < kMaxLimbs - 1; ++p) {
      double carry = __builtin_floor(x[p] * 0x1p-40);
      x[p] = __builtin_fma(-carry, 0x1p40, x[p]);
      x[p + 1] += carry;
    }
  }
  const uint64_t d0 = (uint64_t)x[0], d1 = (uint64_t)x[1], d2 = (uint64_t)x[2],
                 d3 = (uint64_t)x[3];
  const uint64_t w0 = d0 | (d1 << 40);
  const uint64_t w1 = (d1 >> 24) | (d2 << 16) | (d3 << 56);
  const uint64_t w2 = d3 >> 8;
  double out = 0.0;
  if (w0 | w1 | w2) {
    out = round_scaled_words(w0, w1, w2, e_i + f_j);
    if (neg) out = -out;
  }
  *dst = out;
  }
}

}  // namespace

int launch_crt(int64_t m, int64_t n, int r, const void* res, int res_is_i32, int64_t ldr,
               int64_t stride_r, const int32_t* ea, const int32_t* eb, double* c, int64_t ldc,
               hipStream_t s) {
  if (m <= 0 || n <= 0) return OZK_OK;
  const CrtConsts& K = *crt_consts(r);
  dim3 grid((unsigned)((n + 255) / 256), (unsigned)(m < 65535 ? m : 65535));
  if (res_is_i32)
    hipLaunchKernelGGL(crt_kernel<int32_t>, grid, dim3(256), 0, s, m, n,
                       (const int32_t*)res, ldr, stride_r, ea, eb, c, ldc, K);
  else
    hipLaunchKernelGGL(crt_kernel<int8_t>, grid, dim3(256), 0, s, m, n, (const int8_t*)res, ldr,
                       stride_r, ea, eb, c, ldc, K);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

}  // namespace ozk
