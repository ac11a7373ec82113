// Compile-time table of the residue number system: moduli, bit budgets, per-modulus
// residue constants and the Chinese Remainder basis in 2^40 limbs, for r = 1..20.
// Evaluated by the compiler (constexpr), so the same numbers serve host validation and
// device kernels (as __constant__ data) without any run-time initialisation.
//
// [TME4] ("The Missing Fourth Term for the Emulation TME Model: The Residue
// Deconstruction Cost", abstract) names r moduli and a per-output reconstruction but
// neither the moduli nor the formula.  Readings: the greedy pairwise-coprime moduli
// <= 256 (256, 255, 253, 251, ...); the textbook CRT basis
// E_l = (M/m_l) * ((M/m_l)^-1 mod m_l); the budget Q = floor(log2((M-1)/2)).
#pragma once

#include <stdint.h>

namespace ozk {

constexpr int kTableModuli = 20;
constexpr int kTableLimbs = 4;  // 4 x 40 bits >= log2(M) for r <= 20

struct RnsTable {
  int32_t moduli[kTableModuli];
  int32_t q[kTableModuli + 1];                 // Q = floor(log2((M_r - 1)/2))
  int32_t limbs[kTableModuli + 1];             // 40-bit limbs needed for M_r
  double inv[kTableModuli];                    // RN(1/m)
  double c32[kTableModuli];                    // smod(2^32, m)
  double frac[kTableModuli + 1][kTableModuli]; // RN(E_l / M_r) = RN(w_l / m_l)
  double e_limb[kTableModuli + 1][kTableModuli][kTableLimbs];  // E_l, base 2^40
  double m_limb[kTableModuli + 1][kTableLimbs];                // M_r, base 2^40
};

namespace rns_detail {

struct U192 {
  uint32_t w[6];
};

constexpr U192 u192(uint32_t v) {
  U192 x{};
  x.w[0] = v;
  return x;
}

constexpr U192 mul_small(const U192& a, uint32_t b) {
  U192 out{};
  uint64_t carry = 0;
  for (int i = 0; i < 6; ++i) {
    uint64_t t = (uint64_t)a.w[i] * b + carry;
    out.w[i] = (uint32_t)t;
    carry = t >> 32;
  }
  return out;
}

constexpr U192 div_small(const U192& a, uint32_t b) {
  U192 q{};
  uint64_t r = 0;
  for (int i = 5; i >= 0; --i) {
    uint64_t cur = (r << 32) | a.w[i];
    q.w[i] = (uint32_t)(cur / b);
    r = cur % b;
  }
  return q;
}

constexpr uint32_t mod_small(const U192& a, uint32_t b) {
  uint64_t r = 0;
  for (int i = 5; i >= 0; --i) r = ((r << 32) | a.w[i]) % b;
  return (uint32_t)r;
}

constexpr int bit_length(const U192& a) {
  for (int i = 5; i >= 0; --i) {
    if (a.w[i]) {
      int n = 0;
      uint32_t v = a.w[i];
      while (v) {
        ++n;
        v >>= 1;
      }
      return 32 * i + n;
    }
  }
  return 0;
}

constexpr U192 sub_one_half(U192 a) {  // (a - 1) >> 1
  for (int i = 0; i < 6; ++i) {
    if (a.w[i]--) break;
  }
  U192 out{};
  for (int i = 0; i < 6; ++i) {
    uint32_t hi = (i < 5) ? a.w[i + 1] : 0u;
    out.w[i] = (a.w[i] >> 1) | (hi << 31);
  }
  return out;
}

constexpr double limb40(const U192& a, int p) {
  uint64_t v = 0;
  for (int b = 39; b >= 0; --b) {
    int bit = 40 * p + b;
    int word = bit >> 5;
    uint64_t val = word < 6 ? (a.w[word] >> (bit & 31)) & 1u : 0u;
    v = (v << 1) | val;
  }
  return (double)v;  // < 2^40: exact
}

constexpr uint32_t gcd(uint32_t a, uint32_t b) {
  while (b) {
    uint32_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

constexpr uint32_t inverse_mod(uint32_t a, uint32_t m) {
  int64_t t = 0, newt = 1, rr = m, newr = a % m;
  while (newr != 0) {
    int64_t q = rr / newr;
    int64_t tmp = t - q * newt;
    t = newt;
    newt = tmp;
    tmp = rr - q * newr;
    rr = newr;
    newr = tmp;
  }
  return (uint32_t)(t < 0 ? t + m : t);
}

}  // namespace rns_detail

constexpr RnsTable make_rns_table() {
  using namespace rns_detail;
  RnsTable t{};
  int count = 0;
  for (uint32_t cand = 256; count < kTableModuli && cand >= 2; --cand) {
    bool ok = true;
    for (int i = 0; i < count; ++i) ok = ok && gcd(cand, (uint32_t)t.moduli[i]) == 1;
    if (ok) t.moduli[count++] = (int32_t)cand;
  }
  for (int l = 0; l < kTableModuli; ++l) {
    const int64_t m = t.moduli[l];
    t.inv[l] = 1.0 / (double)m;
    const int64_t p32 = ((int64_t)1 << 32) % m;
    t.c32[l] = (double)(((p32 + m / 2) % m) - m / 2);
  }
  for (int r = 1; r <= kTableModuli; ++r) {
    U192 big_m = u192(1);
    for (int l = 0; l < r; ++l) big_m = mul_small(big_m, (uint32_t)t.moduli[l]);
    t.q[r] = bit_length(sub_one_half(big_m)) - 1;
    t.limbs[r] = bit_length(big_m) <= 120 ? 3 : 4;
    for (int p = 0; p < kTableLimbs; ++p) t.m_limb[r][p] = limb40(big_m, p);
    for (int l = 0; l < r; ++l) {
      const uint32_t m = (uint32_t)t.moduli[l];
      const U192 cof = div_small(big_m, m);
      const uint32_t w = inverse_mod(mod_small(cof, m), m);
      const U192 e = mul_small(cof, w);
      t.frac[r][l] = (double)w / (double)m;
      for (int p = 0; p < kTableLimbs; ++p) t.e_limb[r][l][p] = limb40(e, p);
    }
  }
  return t;
}

}  // namespace ozk
