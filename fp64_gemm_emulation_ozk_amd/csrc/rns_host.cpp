// Host-side accessors of the residue number system table (rns_table.h): moduli, bit
// budgets, and the per-r constant blocks passed to the residue and product kernels.
#include <string.h>

#include <mutex>

#include "ozk_internal.h"
#include "rns_table.h"

namespace ozk {
namespace {

constexpr RnsTable kRns = make_rns_table();

}  // namespace

int moduli_list(int r, int32_t* out) {
  if (r < 1 || r > kMaxModuli || !out) return OZK_EINVAL;
  for (int i = 0; i < r; ++i) out[i] = kRns.moduli[i];
  return OZK_OK;
}

int scaling_bits(int r, int64_t k, int* pa, int* pb) {
  if (r < 1 || r > kMaxModuli || k < 1) return OZK_EINVAL;
  if (k > OZK_MAX_K) return OZK_ERANGE;
  int ceil_log2 = 0;
  while ((int64_t(1) << ceil_log2) < k) ++ceil_log2;
  const int beta = kRns.q[r] - ceil_log2;
  if (beta < 2) return OZK_ERANGE;
  // Each width is capped at kWidthCap: it binds only for r = 20 with k <= 2.
  const int a = beta / 2, b = beta - beta / 2;
  if (pa) *pa = a < kWidthCap ? a : kWidthCap;
  if (pb) *pb = b < kWidthCap ? b : kWidthCap;
  return OZK_OK;
}

namespace {

// Unsigned 192-bit integers in three 64-bit words (least significant first), enough for
// 2 (M - 1) < 2^157 and for the products below.
struct W192 {
  uint64_t w[3];
};

W192 w192_mul_small(const W192& a, uint64_t b) {  // a * b, b < 2^32, no overflow here
  W192 out{};
  unsigned __int128 carry = 0;
  for (int i = 0; i < 3; ++i) {
    unsigned __int128 t = (unsigned __int128)a.w[i] * b + carry;
    out.w[i] = (uint64_t)t;
    carry = t >> 64;
  }
  return out;
}

W192 w192_pow2_plus(int e, uint64_t t) {  // 2^e + t, e < 128, t < 2^32
  W192 out{};
  out.w[e / 64] = uint64_t(1) << (e % 64);
  unsigned __int128 lo = (unsigned __int128)out.w[0] + t;
  out.w[0] = (uint64_t)lo;
  if (lo >> 64) {
    if (++out.w[1] == 0) ++out.w[2];
  }
  return out;
}

W192 w192_mul(const W192& a, const W192& b) {  // low 192 bits of a * b
  uint64_t r[6] = {0, 0, 0, 0, 0, 0};
  for (int i = 0; i < 3; ++i) {
    unsigned __int128 carry = 0;
    for (int j = 0; j + i < 6 && j < 3; ++j) {
      unsigned __int128 t = (unsigned __int128)a.w[i] * b.w[j] + r[i + j] + carry;
      r[i + j] = (uint64_t)t;
      carry = t >> 64;
    }
    if (i + 3 < 6) r[i + 3] += (uint64_t)carry;
  }
  return W192{{r[0], r[1], r[2]}};
}

bool w192_le(const W192& a, const W192& b) {
  for (int i = 2; i >= 0; --i)
    if (a.w[i] != b.w[i]) return a.w[i] < b.w[i];
  return true;
}

uint64_t isqrt_u64(uint64_t x) {  // floor(sqrt(x)), x < 2^40 here
  uint64_t r = 0;
  for (uint64_t bit = uint64_t(1) << 20; bit; bit >>= 1)
    if ((r + bit) * (r + bit) <= x) r += bit;
  return r;
}

}  // namespace

int scaling_bits_norm(int r, int64_t k, int* pa, int* pb) {
  if (r < 1 || r > kMaxModuli || k < 1) return OZK_EINVAL;
  if (k > OZK_MAX_K) return OZK_ERANGE;
  // 2 (M - 1) and t = isqrt(k - 1) + 1 >= sqrt(k): the budget holds when
  // (2^(aA+1) + t)(2^(aB+1) + t) <= 2 (M - 1).
  W192 m{{1, 0, 0}};
  for (int l = 0; l < r; ++l) m = w192_mul_small(m, (uint64_t)kRns.moduli[l]);
  if (m.w[0]-- == 0) {
    if (m.w[1]-- == 0) --m.w[2];
  }
  const W192 two_m1 = w192_mul_small(m, 2);
  const uint64_t t = isqrt_u64((uint64_t)k - 1) + 1;
  const int q = kRns.q[r];
  int aa = (q - 1) / 2 < kWidthCap ? (q - 1) / 2 : kWidthCap;
  int ab = q - 1 - (q - 1) / 2 < kWidthCap ? q - 1 - (q - 1) / 2 : kWidthCap;
  while (!w192_le(w192_mul(w192_pow2_plus(aa + 1, t), w192_pow2_plus(ab + 1, t)), two_m1)) {
    if (aa >= ab)
      --aa;
    else
      --ab;
    if (aa < 1 || ab < 1) return OZK_ERANGE;
  }
  if (pa) *pa = aa;
  if (pb) *pb = ab;
  return OZK_OK;
}

int scaling_widths(int scaling, int r, int64_t k, int* wa, int* wb) {
  if (scaling == OZK_SCALING_MAX) return scaling_bits(r, k, wa, wb);
  if (scaling == OZK_SCALING_NORM) return scaling_bits_norm(r, k, wa, wb);
  return OZK_EINVAL;
}

const ResidueConsts* residue_consts(int r, int p_bits) {
  // p_bits selects whether scaled integers may exceed 2^51, the range where the
  // x + 1.5*2^52 rounding and the fp64 quotient are exact (the "wide" split path, exact
  // up to 2^76 = kWidthCap bits).  Widths come from scaling_widths, which never exceeds
  // the cap; a larger p_bits is refused.
  static ResidueConsts table[kMaxModuli + 1][2];
  static std::once_flag once;
  std::call_once(once, [] {
    for (int rr = 1; rr <= kMaxModuli; ++rr) {
      for (int wide = 0; wide < 2; ++wide) {
        ResidueConsts& c = table[rr][wide];
        memset(&c, 0, sizeof c);
        c.r = rr;
        c.wide = wide;
        for (int l = 0; l < rr; ++l) {
          c.m[l] = (double)kRns.moduli[l];
          c.inv[l] = kRns.inv[l];
          c.c32[l] = kRns.c32[l];
        }
      }
    }
  });
  if (r < 1 || r > kMaxModuli || p_bits > kWidthCap) return nullptr;
  return &table[r][p_bits > 51 ? 1 : 0];
}

const CrtConsts* crt_consts(int r) {
  static CrtConsts table[kMaxModuli + 1];
  static std::once_flag once;
  std::call_once(once, [] {
    for (int rr = 1; rr <= kMaxModuli; ++rr) {
      CrtConsts& c = table[rr];
      memset(&c, 0, sizeof c);
      c.r = rr;
      c.limbs = kRns.limbs[rr];
      for (int p = 0; p < kMaxLimbs; ++p) c.m_limb[p] = kRns.m_limb[rr][p];
      for (int l = 0; l < rr; ++l) {
        c.mod[l] = kRns.moduli[l];
        c.inv[l] = kRns.inv[l];
        c.frac[l] = kRns.frac[rr][l];
        for (int p = 0; p < kMaxLimbs; ++p) c.e_limb[l][p] = kRns.e_limb[rr][l][p];
      }
    }
  });
  if (r < 1 || r > kMaxModuli) return nullptr;
  return &table[r];
}

}  // namespace ozk
