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
  if (pa) *pa = beta / 2;
  if (pb) *pb = beta - beta / 2;
  return OZK_OK;
}

const ResidueConsts* residue_consts(int r, int p_bits) {
  // p_bits selects whether scaled integers may exceed 2^51, the range where the
  // x + 1.5*2^52 rounding and the fp64 quotient are exact (the "wide" split path).
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
  if (r < 1 || r > kMaxModuli) return nullptr;
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
