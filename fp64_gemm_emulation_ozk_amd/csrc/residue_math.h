// Per-element arithmetic of the deconstruction: scaled integer and its symmetric
// residues modulo each modulus, produced as bytes.
//
// [TME4] abstract: every streamed fp64 operand is scaled, rounded and reduced modulo
// each of the r moduli on the SIMT pipes.  The fp64 pipe of CDNA runs at full rate, so
// the reduction is done in fp64 with exact arithmetic:
//
//   a' = RNE(a 2^e)                    ldexp is exact here; rint rounds half to even
//   narrow (|a'| <= 2^51):
//     q   = RN(a' * RN(1/m) + 1.5*2^52) - 1.5*2^52     = round(a'/m)  (exact, below)
//     rho = a' - q m                                   = smod(a', m)
//   wide (|a'| <= 2^76):  a' = hi*2^32 + lo, lo in [0, 2^32), |hi| <= 2^44
//     t   = hi * smod(2^32, m) + lo     (|t| <= 2^44 * 127 + 2^32 < 2^51, congruent to
//                                        a' mod m; beyond 2^76 this bound fails)
//     then q and rho as above with t in place of a'.
//   rho is wanted as a byte only, so it is formed modulo 2^32 from the low words of the
//   magic-offset doubles (residue_byte).
//
// Exactness of q: for odd m <= 255 the true quotient t/m is never closer than 1/(2m)
// to a half-integer, while |t * RN(1/m) - t/m| <= |t|/m * 2^-53 <= 1/(4m) < 1/(2m) for
// |t| <= 2^51; so the rounding picks round(t/m) and rho = t - m round(t/m) is the
// symmetric residue in [-(m-1)/2, (m-1)/2].  For m = 256 the residue is the low byte
// of a' in two's complement, i.e. smod(a', 256) in [-128, 127].  Adding 1.5*2^52 to an
// integer |v| < 2^51 stores v + 2^51 in the low mantissa bits, so the low byte of the
// double's bit pattern is v mod 256: no conversion instruction is needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ozk {

__device__ __forceinline__ uint32_t lo32(double x) { return (uint32_t)__double_as_longlong(x); }

// Scaled integer of one element, prepared for the residue loop.
struct Prepared {
  double v;    // narrow: a'        wide: lo
  double vm;   // v + 1.5*2^52
  double hi;   // wide only: floor(a' / 2^32)
};

template <bool kWide>
__device__ __forceinline__ Prepared prepare_element(double a, int e) {
  constexpr double kMagicD = 6755399441055744.0;
  Prepared p;
  double xr = __builtin_rint(__builtin_ldexp(a, e));
  if (kWide) {
    p.hi = __builtin_floor(xr * 0x1p-32);
    p.v = __builtin_fma(-p.hi, 0x1p32, xr);
  } else {
    p.hi = 0.0;
    p.v = xr;
  }
  p.vm = p.v + kMagicD;
  return p;
}

// Low byte of smod(a', m) for an odd modulus m (inv = RN(1/m), c32 = smod(2^32, m)).
// Only the byte is needed, so the residue is formed modulo 2^32 in integer arithmetic:
// with q = round(t / m) (t = a' narrow, t = hi c32 + lo wide, |t| <= 2^51), the low words
// of q + 1.5*2^52 and t + 1.5*2^52 are q and t modulo 2^32, and the low byte of
// t - q m is that of their combination by one signed 24-bit multiply-add (only the low 24
// bits of q matter modulo 2^8).  Narrow: one fp64 FMA and one integer operation per
// modulus; wide: three fp64 operations (t + 1.5*2^52 exact by FMA, then t, then q).
template <bool kWide>
__device__ __forceinline__ uint32_t residue_byte(const Prepared& p, double m, double inv,
                                                 double c32) {
  constexpr double kMagicD = 6755399441055744.0;
  const int neg_m = -(int)m;
  if (kWide) {
    const double tm = __builtin_fma(p.hi, c32, p.vm);   // t + 1.5*2^52, exact
    const double qm = __builtin_fma(tm - kMagicD, inv, kMagicD);
    return (uint32_t)(__mul24((int)lo32(qm), neg_m) + (int)lo32(tm));
  } else {
    const double qm = __builtin_fma(p.v, inv, kMagicD);
    return (uint32_t)(__mul24((int)lo32(qm), neg_m) + (int)lo32(p.vm));
  }
}

// Byte of the m = 256 residue: the low byte of a' (wide: of lo, since 2^32 = 0 mod 256).
__device__ __forceinline__ uint32_t residue_byte_256(const Prepared& p) { return lo32(p.vm); }

__device__ __forceinline__ uint32_t pack4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);   // b0.byte0, b1.byte0
  uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);          // lo.b0, lo.b1, hi.b0, hi.b1
}

// Exponent of a line from the bit pattern of its largest |x| (max rule).
__device__ __forceinline__ int line_exponent(uint64_t maxbits, int p_bits) {
  if (maxbits >= 0x7ff0000000000000ull) return INT32_MIN;      // Inf or NaN in the line
  if (maxbits == 0) return 0;
  double t = __longlong_as_double((long long)maxbits);
  return p_bits - __builtin_amdgcn_frexp_exp(t);               // p - 1 - ilogb(t)
}

// Norm rule (tighter row/column scaling): the exponent of a line from the bit pattern of
// its largest |x| and s = sum over the line of (x 2^-T)^2, T = ilogb(max |x|), summed in
// fp64 in a fixed order.  s >= 1 (the largest term is in [1, 4)) and its relative error
// is below 2^-35 for lines of at most 2^17 entries, so RN(s (1 + 2^-32)) bounds the exact
// sum from above and, with u = its ilogb, ||x||_2 < 2^(T + floor(u/2) + 1):
// e = alpha - 1 - (T + floor(u/2)) keeps 2^e ||x||_2 < 2^alpha.
__device__ __forceinline__ int norm_exponent(uint64_t maxbits, double s, int alpha) {
  if (maxbits >= 0x7ff0000000000000ull) return INT32_MIN;     // Inf or NaN in the line
  if (maxbits == 0) return 0;
  const int t = __builtin_amdgcn_frexp_exp(__longlong_as_double((long long)maxbits)) - 1;
  const int u = __builtin_amdgcn_frexp_exp(s * (1.0 + 0x1p-32)) - 1;
  return alpha - 1 - (t + (u >> 1));
}

// (x 2^-T)^2 added to acc, T = ilogb of the line's maximum (0 when that is 0 or not
// finite: the sum is then unused).
__device__ __forceinline__ int line_ilogb(uint64_t maxbits) {
  if (maxbits == 0 || maxbits >= 0x7ff0000000000000ull) return 0;
  return __builtin_amdgcn_frexp_exp(__longlong_as_double((long long)maxbits)) - 1;
}

__device__ __forceinline__ uint64_t abs_bits(double x) {
  return (uint64_t)__double_as_longlong(x) & 0x7fffffffffffffffull;
}

}  // namespace ozk
