// Host-side constants of the residue number system: moduli, bit budgets, per-modulus
// residue constants and the CRT basis in 2^40 limbs.  Built once per r (thread-safe
// function-local statics) and passed to kernels by value.
//
// [TME4] ("The Missing Fourth Term for the Emulation TME Model: The Residue
// Deconstruction Cost", abstract) names r moduli and a per-output reconstruction but
// neither the moduli nor the formula.  Here: the greedy pairwise-coprime moduli <= 256,
// the textbook Chinese Remainder basis E_l = (M/m_l) * ((M/m_l)^-1 mod m_l), and the
// budget Q = floor(log2((M-1)/2)), beta = Q - ceil(log2 k), P_A = floor(beta/2),
// P_B = beta - P_A, which keeps every exact dot product inside (-(M-1)/2, (M-1)/2).
#include <math.h>
#include <string.h>

#include <mutex>

#include "ozk_internal.h"

namespace ozk {
namespace {

// Unsigned 192-bit integer, six little-endian 32-bit words.
struct U192 {
  uint32_t w[6];
};

U192 u192_from(uint32_t v) {
  U192 x;
  memset(&x, 0, sizeof x);
  x.w[0] = v;
  return x;
}

U192 mul_small(const U192& a, uint32_t b) {
  U192 out;
  uint64_t carry = 0;
  for (int i = 0; i < 6; ++i) {
    uint64_t t = (uint64_t)a.w[i] * b + carry;
    out.w[i] = (uint32_t)t;
    carry = t >> 32;
  }
  return out;  // caller guarantees no overflow (M < 2^160)
}

U192 div_small(const U192& a, uint32_t b, uint32_t* rem) {
  U192 q;
  uint64_t r = 0;
  for (int i = 5; i >= 0; --i) {
    uint64_t cur = (r << 32) | a.w[i];
    q.w[i] = (uint32_t)(cur / b);
    r = cur % b;
  }
  if (rem) *rem = (uint32_t)r;
  return q;
}

int bit_length(const U192& a) {
  for (int i = 5; i >= 0; --i)
    if (a.w[i]) return 32 * i + 32 - __builtin_clz(a.w[i]);
  return 0;
}

U192 sub_one(U192 a) {
  for (int i = 0; i < 6; ++i) {
    if (a.w[i]--) break;
  }
  return a;
}

U192 shr1(const U192& a) {
  U192 out;
  for (int i = 0; i < 6; ++i) {
    uint32_t hi = (i < 5) ? a.w[i + 1] : 0;
    out.w[i] = (a.w[i] >> 1) | (hi << 31);
  }
  return out;
}

// Bits [40*p, 40*p + 40) of a as a double (exact).
double limb40(const U192& a, int p) {
  double v = 0.0;
  for (int b = 39; b >= 0; --b) {
    int bit = 40 * p + b;
    int word = bit >> 5;
    uint32_t val = word < 6 ? (a.w[word] >> (bit & 31)) & 1u : 0u;
    v = 2.0 * v + (double)val;
  }
  return v;
}

uint32_t gcd_u32(uint32_t a, uint32_t b) {
  while (b) {
    uint32_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// Modular inverse of a mod m (a, m coprime) by the extended Euclidean algorithm.
uint32_t inverse_mod(uint32_t a, uint32_t m) {
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
  if (t < 0) t += m;
  return (uint32_t)t;
}

struct Tables {
  int32_t moduli[kMaxModuli];
  int q[kMaxModuli + 1];                  // Q for r = index
  CrtConsts crt[kMaxModuli + 1];
};

const Tables& tables() {
  static Tables t;
  static std::once_flag once;
  std::call_once(once, [] {
    int count = 0;
    for (uint32_t cand = 256; count < kMaxModuli && cand >= 2; --cand) {
      bool ok = true;
      for (int i = 0; i < count; ++i) ok = ok && gcd_u32(cand, (uint32_t)t.moduli[i]) == 1;
      if (ok) t.moduli[count++] = (int32_t)cand;
    }
    for (int r = 1; r <= kMaxModuli; ++r) {
      U192 big_m = u192_from(1);
      for (int l = 0; l < r; ++l) big_m = mul_small(big_m, (uint32_t)t.moduli[l]);
      // Q = floor(log2((M - 1) / 2)) = bit_length((M-1)/2) - 1
      t.q[r] = bit_length(shr1(sub_one(big_m))) - 1;
      CrtConsts& c = t.crt[r];
      memset(&c, 0, sizeof c);
      c.r = r;
      c.limbs = bit_length(big_m) <= 120 ? 3 : 4;
      for (int p = 0; p < kMaxLimbs; ++p) c.m_limb[p] = limb40(big_m, p);
      for (int l = 0; l < r; ++l) {
        uint32_t m = (uint32_t)t.moduli[l];
        uint32_t cof_mod = 0;
        U192 cof = div_small(big_m, m, nullptr);
        div_small(cof, m, &cof_mod);
        uint32_t w = inverse_mod(cof_mod, m);
        U192 e = mul_small(cof, w);
        c.mod[l] = (int32_t)m;
        c.inv[l] = 1.0 / (double)m;
        c.frac[l] = (double)w / (double)m;
        for (int p = 0; p < kMaxLimbs; ++p) c.e_limb[l][p] = limb40(e, p);
      }
    }
  });
  return t;
}

}  // namespace

int moduli_list(int r, int32_t* out) {
  if (r < 1 || r > kMaxModuli || !out) return OZK_EINVAL;
  const Tables& t = tables();
  for (int i = 0; i < r; ++i) out[i] = t.moduli[i];
  return OZK_OK;
}

int scaling_bits(int r, int64_t k, int* pa, int* pb) {
  if (r < 1 || r > kMaxModuli || k < 1) return OZK_EINVAL;
  if (k > OZK_MAX_K) return OZK_ERANGE;
  int ceil_log2 = 0;
  while ((int64_t(1) << ceil_log2) < k) ++ceil_log2;
  int beta = tables().q[r] - ceil_log2;
  if (beta < 2) return OZK_ERANGE;
  if (pa) *pa = beta / 2;
  if (pb) *pb = beta - beta / 2;
  return OZK_OK;
}

const ResidueConsts* residue_consts(int r, int p_bits) {
  // One table per (r, wide); p_bits only selects whether scaled integers may exceed
  // 2^51, the range where x + 1.5*2^52 rounding and the fp64 quotient are exact.
  static ResidueConsts table[kMaxModuli + 1][2];
  static std::once_flag once;
  std::call_once(once, [] {
    const Tables& t = tables();
    for (int r = 1; r <= kMaxModuli; ++r) {
      for (int wide = 0; wide < 2; ++wide) {
        ResidueConsts& c = table[r][wide];
        memset(&c, 0, sizeof c);
        c.r = r;
        c.wide = wide;
        for (int l = 0; l < r; ++l) {
          int32_t m = t.moduli[l];
          c.m[l] = (double)m;
          c.inv[l] = 1.0 / (double)m;
          int64_t p32 = ((int64_t)1 << 32) % m;          // 2^32 mod m
          int64_t h = m / 2;
          c.c32[l] = (double)(((p32 + h) % m) - h);      // symmetric representative
        }
      }
    }
  });
  if (r < 1 || r > kMaxModuli) return nullptr;
  return &table[r][p_bits > 51 ? 1 : 0];
}

const CrtConsts* crt_consts(int r) {
  if (r < 1 || r > kMaxModuli) return nullptr;
  return &tables().crt[r];
}

}  // namespace ozk
