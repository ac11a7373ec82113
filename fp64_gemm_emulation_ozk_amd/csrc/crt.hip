// CRT reconstruction and inverse scaling: the per-output reconstruction term of Ozaki
// scheme II ([TME4] abstract).
//
// Given symmetric residues c_l (|c_l| <= 128) of the exact integer X modulo m_l, with
// |X| <= 2^Q <= (M-1)/2:
//   1. the digit sums S_b = sum_l c_l e_lb of the basis E_l in balanced base 256, and the
//      same for the 24-bit fractions F_l ~ 2^24 E_l / M, come from one int8 matrix-core
//      product per 32 outputs (crt_kernel below);
//   2. q = rint(2^-24 sum_l c_l F_l) is exact (the distance of sum_l c_l E_l / M to the
//      integer q is at most 1/2 - 2^Q/M, and 1/2 - 2^Q/M >= 0.0142 for every r <= 20);
//   3. X = sum_b S_b 256^b - q M in 2^40 limbs held in fp64: every limb sum stays below
//      2^52, so all fp64 operations are exact;
//   4. limbs are normalised to digits in [0, 2^40), the sign left in the top digit;
//      RN(X 2^-s) is formed with one fp64 rounding of the folded top digits plus an exact
//      tie correction (round_fast), or, for a result below the normal range, by splitting
//      off the sign and rounding the magnitude at the reduced precision (round_exact), so
//      the output is rounded exactly once.
// The constants come from compile-time tables in __constant__ memory.
#include "ozk_internal.h"
#include "rns_table.h"

namespace ozk {

__constant__ RnsTable d_rns = make_rns_table();

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

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

// The carry pass: digits 0..L-2 of X = sum_p x[p] 2^(40 p) (|x[p]| < 2^52) brought into
// [0, 2^40), the sign carried into the top limb x[L-1].
template <int L>
__device__ __forceinline__ void carry_digits(double (&x)[4]) {
#pragma unroll
  for (int p = 0; p < L - 1; ++p) {
    const double carry = __builtin_floor(x[p] * 0x1p-40);
    x[p] = __builtin_fma(-carry, 0x1p40, x[p]);
    x[p + 1] += carry;
  }
}

// RN(X 2^-s) exactly for any X in carried digits (the path of small results): the sign
// is split off, the magnitude carried again and rounded by round_digits, which also
// rounds subnormal results at their reduced precision.
template <int L>
__device__ __forceinline__ double round_exact(const double (&xin)[4], int s) {
  double x[4] = {xin[0], xin[1], xin[2], xin[3]};
  const bool neg = x[L - 1] < 0.0;
  if (neg) {
#pragma unroll
    for (int p = 0; p < L; ++p) x[p] = -x[p];
    carry_digits<L>(x);
  }
  const double o = round_digits<L>(x, s);
  return neg ? -o : o;
}

// The double next to v (finite, nonzero) in the direction of +Inf.
__device__ __forceinline__ double next_up(double v) {
  const int64_t b = __double_as_longlong(v);
  return __longlong_as_double(b + (v > 0.0 ? 1 : -1));
}

// RN(X 2^-s) for X in carried digits, both signs at once, for results in the normal
// range.  With B = 2^40 and the lower digits non-negative, the digits are folded from the
// top, v <- v B + d, which stays exact while the folded value v lies in [-8192, 8192)
// (then |v B + d| <= 2^53).  The first level whose v is outside that range gives
// S = RN(v B + d) with |S| >= 2^53, so S has at least 54 bits and every rounding
// midpoint is an integer; the digits below add 0 <= eps < 1 unit, which moves the true
// value towards +Inf and decides only when v B + d lies exactly on the midpoint above S:
// then the result is the next double above S.  If no level is outside the range the
// fold reaches the last digit and S = RN(X) directly.  kBigTop: the top digit can leave
// [-8192, 8192) at this r (the budget bounds |X| <= 2^(Q+1)).
template <int L, bool kBigTop>
__device__ __forceinline__ double round_fast(const double (&d)[4], int s) {
  constexpr double B = 0x1p40;
  double hv, lv;
  bool below;
  int base;
  auto big = [](double v) { return v >= 8192.0 || v < -8192.0; };
  if constexpr (L == 1) {
    hv = 0.0; lv = d[0]; below = false; base = 0;
  } else if constexpr (L == 2) {
    hv = d[1]; lv = d[0]; below = false; base = 0;
  } else if constexpr (L == 3) {
    const bool ba = kBigTop && big(d[2]);
    const double b = __builtin_fma(d[2], B, d[1]);
    hv = ba ? d[2] : b;
    lv = ba ? d[1] : d[0];
    below = ba && d[0] != 0.0;
    base = ba ? 40 : 0;
  } else {
    const bool ba = kBigTop && big(d[3]);
    const double b = __builtin_fma(d[3], B, d[2]);
    const bool bb = big(b);
    const double c = __builtin_fma(b, B, d[1]);
    hv = ba ? d[3] : (bb ? b : c);
    lv = ba ? d[2] : (bb ? d[1] : d[0]);
    below = ba ? (d[1] != 0.0 || d[0] != 0.0) : (bb && d[0] != 0.0);
    base = ba ? 80 : (bb ? 40 : 0);
  }
  double S = __builtin_fma(hv, B, lv);
  const double err = __builtin_fma(hv, B, -S) + lv;   // exact: an integer below 2^42
  const double up = next_up(S);
  if (below && err == 0.5 * (up - S)) S = up;
  return __builtin_ldexp(S, base - s);
}

// Carries and the single rounding of X = sum_p x[p] 2^(40 p) (|x[p]| < 2^52, L limbs):
// the fast signed rounding, and the exact path for results below 2^-1021 in magnitude
// (subnormal, zero or underflowing), which only the lanes holding one take.
template <int L, bool kBigTop>
__device__ __forceinline__ double finish(double (&x)[4], int s, bool nan) {
  carry_digits<L>(x);
  double o = round_fast<L, kBigTop>(x, s);
  if (__builtin_fabs(o) < 0x1p-1021) o = round_exact<L>(x, s);
  return nan ? __builtin_nan("") : o;
}

// ---------------------------------------------------------------- CRT on the matrix cores
// The lift sum_l c_l E_l is a product of the residue matrix (outputs x r) with the basis
// (r x digits): E_l is written in balanced base-256 digits e_lb in [-128, 127] (the bytes
// of E_l + 0x80..80, minus 128), so
//   S_b = sum_l c_l e_lb   (|S_b| <= 20 * 2^14, exact in int32)
// is one v_mfma_i32_32x32x32_i8 per 32 outputs with the digits as the A operand (row b)
// and the residues as the B operand (column = output).  Four more rows hold the balanced
// digits of F_l = RN(2^24 w_l / m_l) (E_l / M = w_l / m_l), from which
//   q = rint(2^-24 sum_l c_l F_l)
// is exact: the rows' rounding adds at most 20 * 128 * 2^-25 < 1e-4 to the exact
// sum_l c_l E_l / M = q + X / M, whose distance to q is at most 1/2 - 0.0142.  Then
//   X = sum_b S_b 256^b - q M
// in 2^40 limbs (five digits per limb: every limb sum stays below 2^52, exact in fp64).
//
// Output layout of the MFMA: lane i holds column i % 32 and, in register v, row
// 8 (v / 4) + 4 (i / 32) + v % 4.  Two MFMAs (outputs j0 .. j0+31 and j0+32 .. j0+63)
// followed by v_permlane32_swap on each register pair leave lane i with every row of
// output j0 + i.  The K slots of A and B pair up by (lane half, register, byte); residue
// of modulus l sits in half l / H, byte l % H (H = ceil(r / 2)), the rest are zero.
struct CrtDigitTable {
  int8_t a[kTableModuli + 1][64][16];  // A operand per r and lane
  int32_t ne[kTableModuli + 1];        // balanced E digits per r
};

constexpr CrtDigitTable make_crt_digit_table() {
  using namespace rns_detail;
  CrtDigitTable t{};
  const RnsTable base = make_rns_table();
  for (int r = 1; r <= kTableModuli; ++r) {
    U192 big_m = u192(1);
    for (int l = 0; l < r; ++l) big_m = mul_small(big_m, (uint32_t)base.moduli[l]);
    const int ne = (bit_length(big_m) + 1 + 7) / 8;   // E_l + 0x80..80 < 256^ne
    t.ne[r] = ne;
    const int h_per = (r + 1) / 2;
    for (int l = 0; l < r; ++l) {
      const uint32_t m = (uint32_t)base.moduli[l];
      const U192 cof = div_small(big_m, m);
      const uint32_t w = inverse_mod(mod_small(cof, m), m);
      U192 e = mul_small(cof, w);
      // + 0x80 in each of the ne bytes
      uint64_t carry = 0;
      for (int i = 0; i < 6; ++i) {
        uint32_t add = 0;
        for (int by = 0; by < 4; ++by)
          if (4 * i + by < ne) add |= 0x80u << (8 * by);
        const uint64_t v = (uint64_t)e.w[i] + add + carry;
        e.w[i] = (uint32_t)v;
        carry = v >> 32;
      }
      // F_l = RN(2^24 w / m) (m = 256: exact), + 0x80808080
      const uint64_t f = (((uint64_t)w << 25) / m + 1) >> 1;
      const uint64_t fb = f + 0x80808080ull;
      const int half = l / h_per, slot = l % h_per;
      for (int row = 0; row < 32; ++row) {
        int digit = 0;
        if (row < ne)
          digit = (int)((e.w[row / 4] >> (8 * (row % 4))) & 0xffu) - 128;
        else if (row < ne + 4)
          digit = (int)((fb >> (8 * (row - ne))) & 0xffu) - 128;
        t.a[r][row + 32 * half][slot] = (int8_t)digit;
      }
    }
  }
  return t;
}

__constant__ CrtDigitTable d_crt = make_crt_digit_table();
constexpr CrtDigitTable kCrtDigits = make_crt_digit_table();

template <int R>
struct CrtShape {
  static constexpr int kH = (R + 1) / 2;             // moduli per lane half
  static constexpr int kNE = kCrtDigits.ne[R];       // E digit rows
  static constexpr int kRows = kNE + 4;              // + F digit rows
  static constexpr int kL = (kNE + 4) / 5;           // 2^40 limbs of X
  static constexpr int kSwaps = ((kRows + 7) / 8) * 4;  // registers holding used rows
  // |X| < 2^(Q+1): the top carried digit lies in [-8192, 8192) unless Q + 1 exceeds the
  // top limb's position by more than 13 bits
  static constexpr bool kBigTop = kL >= 3 && make_rns_table().q[R] + 1 - 40 * (kL - 1) > 13;
};

// Symmetric residue of one input value of modulus l (int8 residues pass through).
template <typename T>
__device__ __forceinline__ uint32_t residue_byte(T v, int l) {
  if (sizeof(T) == 1) return (uint32_t)(uint8_t)v;
  const int mod = d_rns.moduli[l];
  if (mod == 256) return (uint32_t)(v & 0xff);
  constexpr double kMagicD = 6755399441055744.0;
  const double d = (double)v;
  const double q = __builtin_fma(d, d_rns.inv[l], kMagicD) - kMagicD;
  return (uint32_t)((int)__builtin_fma(-q, (double)mod, d) & 0xff);
}

// B operands of a group from byte loads (any alignment, ragged tails, int32 inputs):
// lane (half, col) gathers the residues of outputs j0 + col and j0 + 32 + col for the
// moduli of its half.  Every lane loads from a valid address (column clamped to n - 1,
// modulus to r - 1) and zeroes what lies outside, so the loads need no branches.
template <int R, typename T>
__device__ __forceinline__ void load_b_bytes(const T* __restrict__ src, int64_t stride_r,
                                             int64_t j0, int64_t n, int half, int col,
                                             v4i& b1v, v4i& b2v) {
  using S = CrtShape<R>;
  const int64_t ja = j0 + col < n ? j0 + col : n - 1;
  const int64_t jb = j0 + 32 + col < n ? j0 + 32 + col : n - 1;
  const bool va = j0 + col < n, vb = j0 + 32 + col < n;
  uint32_t w1[4] = {0u, 0u, 0u, 0u}, w2[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int slot = 0; slot < S::kH; ++slot) {
    const int l0 = half * S::kH + slot;
    const bool vl = l0 < R;
    const int l = vl ? l0 : R - 1;
    const T* p = src + l * stride_r;
    const uint32_t b1 = residue_byte<T>(p[ja], l);
    const uint32_t b2 = residue_byte<T>(p[jb], l);
    w1[slot / 4] |= (vl && va ? b1 : 0u) << (8 * (slot % 4));
    w2[slot / 4] |= (vl && vb ? b2 : 0u) << (8 * (slot % 4));
  }
  b1v = v4i{(int)w1[0], (int)w1[1], (int)w1[2], (int)w1[3]};
  b2v = v4i{(int)w2[0], (int)w2[1], (int)w2[2], (int)w2[3]};
}

// B operands of a whole group of 64 int8 residues from dword loads (4-byte aligned
// rows and planes): in each quad of lanes (col = 4t + u), lane u loads the four outputs
// 4t .. 4t+3 of modulus (half H + 4d + u) for the first and second 32 outputs (k), and a
// 4 x 4 byte transpose across the quad (two DPP exchanges, two byte permutes) leaves
// lane u with the four moduli of output 4t + u, which is dword d of its B operand.  The
// loads and the transposes are separate steps so that several groups' loads can be in
// flight before the first transpose waits for its data.
template <int R>
struct WordLoads {
  static constexpr int kND = (CrtShape<R>::kH + 3) / 4;
  uint32_t w[2][kND];
};

template <int R>
__device__ __forceinline__ void load_words(const int8_t* __restrict__ src, int64_t stride_r,
                                           int half, int t, int u, WordLoads<R>& raw) {
  using S = CrtShape<R>;
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int d = 0; d < WordLoads<R>::kND; ++d) {
      const int slot = 4 * d + u;
      const int l0 = half * S::kH + slot;
      const bool ok = slot < S::kH && l0 < R;
      const int l = ok ? l0 : R - 1;
      const uint32_t x = *reinterpret_cast<const uint32_t*>(src + l * stride_r + 32 * k + 4 * t);
      raw.w[k][d] = ok ? x : 0u;
    }
}

template <int R>
__device__ __forceinline__ void transpose_words(const WordLoads<R>& raw, uint32_t sel1,
                                                uint32_t sel2, v4i& b1v, v4i& b2v) {
  uint32_t w[2][4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int d = 0; d < WordLoads<R>::kND; ++d) {
      const uint32_t x = raw.w[k][d];
      const uint32_t z = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4e, 0xf, 0xf, true);
      const uint32_t s1 = __builtin_amdgcn_perm(z, x, sel1);
      const uint32_t z2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0xb1, 0xf, 0xf, true);
      w[k][d] = __builtin_amdgcn_perm(z2, s1, sel2);
    }
  b1v = v4i{(int)w[0][0], (int)w[0][1], (int)w[0][2], (int)w[0][3]};
  b2v = v4i{(int)w[1][0], (int)w[1][1], (int)w[1][2], (int)w[1][3]};
}

// Persistent waves: each takes groups of 64 consecutive outputs of one row, lane i
// finishing output j0 + i; consecutive waves take consecutive groups.
// Columns past n read as residue 0 and are not stored.
template <int R, typename T>
__global__ __launch_bounds__(256) void crt_kernel(int64_t m, int64_t n, const T* __restrict__ res,
                                                  int64_t ldr, int64_t stride_r,
                                                  const int32_t* __restrict__ ea,
                                                  const int32_t* __restrict__ eb,
                                                  double* __restrict__ c, int64_t ldc) {
  using S = CrtShape<R>;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, col = lane & 31, t = col >> 2, u = col & 3;
  // byte selectors of the quad transpose (see load_b_words)
  const uint32_t sel1 = u < 2 ? 0x05040100u : 0x03020706u;
  const uint32_t sel2 = (u & 1) ? 0x03070105u : 0x06020400u;
  const v4i a_op = *reinterpret_cast<const v4i*>(&d_crt.a[R][lane][0]);
  const int64_t ngroups_row = (n + 63) / 64;
  const int64_t groups = m * ngroups_row;
  const int64_t waves = (int64_t)gridDim.x * 4;
  const bool words = sizeof(T) == 1 &&
                     ((ldr | stride_r | (int64_t)reinterpret_cast<uintptr_t>(res)) & 3) == 0;
  double m_limb[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) m_limb[p] = d_rns.m_limb[R][p];

  // A group covers outputs j0 .. j0+63 of row i; (i, j0) are wave-uniform and advance
  // without divisions.
  auto word_path = [&](int64_t j0) { return words && j0 + 64 <= n; };
  auto finish_group = [&](int64_t i, int64_t j0, const v4i& b1v, const v4i& b2v) {
    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const v16i d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_op, b1v, zero, 0, 0, 0);
    const v16i d2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_op, b2v, zero, 0, 0, 0);
    int sum[S::kRows];
#pragma unroll
    for (int v = 0; v < S::kSwaps; ++v) {
      const auto sw = __builtin_amdgcn_permlane32_swap((unsigned)d1[v], (unsigned)d2[v], false,
                                                       false);
      const int row_a = 8 * (v / 4) + v % 4;      // rows of the first register
      if (row_a < S::kRows) sum[row_a] = (int)sw[0];
      if (row_a + 4 < S::kRows) sum[row_a + 4] = (int)sw[1];
    }
    // q from the F rows, then X in 2^40 limbs.
    // Adjacent digit sums are first combined in int32 (|S_b + 256 S_b+1| < 2^27), which
    // halves the conversions to fp64.
    const int f01 = sum[S::kNE] + 256 * sum[S::kNE + 1];
    const int f23 = sum[S::kNE + 2] + 256 * sum[S::kNE + 3];
    const double tq = __builtin_fma((double)f23, 0x1p16, (double)f01);
    const double q = __builtin_rint(tq * 0x1p-24);
    double x[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int p = 0; p < S::kL; ++p) x[p] = -q * m_limb[p];   // |q| < 2^11.4: exact
#pragma unroll
    for (int b = 0; b < S::kNE; ++b) {
      const int pos = b % 5;           // digit position inside its 2^40 limb
      if (pos == 1 || pos == 3) continue;  // folded into the digit below
      const int v = (pos != 4 && b + 1 < S::kNE) ? sum[b] + 256 * sum[b + 1] : sum[b];
      x[b / 5] = __builtin_fma((double)v, (double)(1ll << (8 * pos)), x[b / 5]);
    }
    const int64_t j = j0 + lane;
    if (j < n) {
      const int32_t e_i = ea[i], f_j = eb[j];
      const bool nan = e_i == INT32_MIN || f_j == INT32_MIN;
      c[i * ldc + j] = finish<S::kL, S::kBigTop>(x, e_i + f_j, nan);
    }
  };
  // Position (row, group within the row) of a group, advanced by `waves` groups.
  struct Pos {
    int64_t i, jg;
  };
  const int64_t g0 = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int64_t adv_i = waves / ngroups_row, adv_j = waves - adv_i * ngroups_row;
  auto advance = [&](Pos p) {
    p.i += adv_i;
    p.jg += adv_j;
    if (p.jg >= ngroups_row) {
      p.jg -= ngroups_row;
      ++p.i;
    }
    return p;
  };
  // Groups per iteration.  One keeps the wave's loads next to its neighbours' (waves
  // take consecutive groups), so the loads in flight chip-wide span few DRAM pages:
  // 8192^2, r = 16, inside the DGEMM step: 449 us with 4 groups per iteration, 433 with
  // 3, 423 with 2, 412 with 1.
  constexpr int kG = 1;
  Pos p{g0 / ngroups_row, g0 - (g0 / ngroups_row) * ngroups_row};
  for (int64_t g = g0; g < groups; g += kG * waves) {
    Pos pos[kG];
    WordLoads<R> raw[kG];
    pos[0] = p;
#pragma unroll
    for (int q = 1; q < kG; ++q) pos[q] = advance(pos[q - 1]);
    p = advance(pos[kG - 1]);
    // issue every word load of the iteration first
#pragma unroll
    for (int q = 0; q < kG; ++q)
      if (g + q * waves < groups && word_path(pos[q].jg * 64))
        load_words<R>(reinterpret_cast<const int8_t*>(res + pos[q].i * ldr) + pos[q].jg * 64,
                      stride_r, half, t, u, raw[q]);
#pragma unroll
    for (int q = 0; q < kG; ++q) {
      if (g + q * waves >= groups) break;           // wave-uniform
      const int64_t i = pos[q].i, j0 = pos[q].jg * 64;
      v4i b1v, b2v;
      if (word_path(j0))
        transpose_words<R>(raw[q], sel1, sel2, b1v, b2v);
      else
        load_b_bytes<R, T>(res + i * ldr, stride_r, j0, n, half, col, b1v, b2v);
      finish_group(i, j0, b1v, b2v);
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
  // Persistent waves (4 per block), each over groups of 64 outputs of a row, at most
  // 16384 blocks (about ten rounds of the chip's resident waves, six per SIMD): inside
  // the DGEMM step at r = 16, 8192^2 takes 422 / 412 / 402 / 395 us with 4096 / 8192 /
  // 16384 / 32768 blocks, 4096^2 106 / 106 / 106 / 113 us (its last round fills badly).
  const int64_t groups = m * ((n + 63) / 64);
  const int64_t want = (groups + 3) / 4;
  const int64_t blocks = want < 16384 ? want : 16384;
  dim3 grid((unsigned)blocks);
  Dispatch<1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20>::go(
      r, grid, s, m, n, res, res_is_i32, ldr, stride_r, ea, eb, c, ldc);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

}  // namespace ozk
