// Emulated fp64 GEMV and low-batch GEMV (Y = A X, X with 1..32 columns): the memory-bound
// case of [TME4] abstract, in its two forms:
//   stored      A arrives as precomputed int8 residue planes (r bytes per element): the
//               deconstruction cost has moved into HBM traffic.
//   on the fly  A arrives as fp64 (8 bytes per element) and every element is scaled,
//               rounded and reduced modulo each modulus in registers before the products:
//               the per-input deconstruction term sits on the VALU.
// Both write the symmetric residues of the exact int32 products; the CRT kernel then
// reconstructs Y.  The stored path feeds v_mfma_i32_32x32x32_i8 with the 1..32
// right-hand sides padded to 32 columns (the MFMA time stays far below the HBM time):
// for K chunk k0 of 32, lane (row or column = lane & 31, half = lane >> 5) supplies the
// 16 bytes at K = k0 + 16*half .. +15, identically for A (rows) and X (columns), so the
// K order inside the instruction does not matter.  The on-the-fly path uses 16-row tiles
// (v_mfma_i32_16x16x32_i8, see there) to keep its accumulators small.
#include <type_traits>

#include "ozk_internal.h"
#include "residue_math.h"
#include "rns_table.h"

namespace ozk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

struct GemvModuli {
  int32_t mod[kMaxModuli];
  double inv[kMaxModuli];
};

__device__ __forceinline__ int sym_residue32(int v, int m, double inv) {
  if (m == 256) return (int)(int8_t)(v & 0xff);
  constexpr double kMagicD = 6755399441055744.0;
  const double d = (double)v;
  const double q = __builtin_fma(d, inv, kMagicD) - kMagicD;
  return (int)__builtin_fma(-q, (double)m, d);
}

// Residues of one 32 x 32 accumulator tile (rows row0.., columns 0..31) to res.
__device__ __forceinline__ void store_tile(const v16i& acc, int lane, int64_t row0, int64_t m,
                                           int nrhs, int mod, double inv, int8_t* res) {
  const int col = lane & 31;
  if (col >= nrhs) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t row = row0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (row < m) res[row * nrhs + col] = (int8_t)sym_residue32(acc[v], mod, inv);
  }
}

// ------------------------------------------------------------------ stored planes
// grid (ceil(m / (128 TR)), r); 4 waves, each TR tiles of 32 rows of one modulus over all
// of K, so every X fragment (read from L2) feeds TR MFMAs.  Per step of 4 K chunks a lane
// loads 64 contiguous bytes of each of its rows (one 128-byte line per row and lane pair);
// the next step's loads are issued before this step's MFMAs.
template <int TR>
__global__ __launch_bounds__(256) void gemv_stored_kernel(
    const int8_t* __restrict__ ap, int64_t lda_p, int64_t a_stride, int64_t m,
    const int8_t* __restrict__ xp, int64_t kp, int64_t x_stride, int nrhs,
    int8_t* __restrict__ res, int64_t res_stride, GemvModuli E) {
  const int l = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 32 * TR;
  if (row0 >= m) return;
  const int half = lane >> 5;
  const int8_t* pa[TR];
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    int64_t row = row0 + 32 * t + (lane & 31);
    row = row < m ? row : m - 1;
    pa[t] = ap + l * a_stride + row * lda_p + 16 * half;
  }
  int col = lane & 31;
  col = col < nrhs ? col : nrhs - 1;
  const int8_t* px = xp + l * x_stride + col * kp + 16 * half;
  v16i acc[TR];
#pragma unroll
  for (int t = 0; t < TR; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0;
  // Register double buffering: the loads of step c + kU are in flight while the MFMAs of
  // step c run.
  constexpr int kU = 4;   // K chunks of 32 bytes per step
  const int64_t nc = kp / 32;
  const int64_t nsteps = nc / kU;
  v4i a0[TR][kU], x0[kU], a1[TR][kU], x1[kU];
  auto load = [&](v4i (&av)[TR][kU], v4i (&xv)[kU], int64_t c) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
      for (int t = 0; t < TR; ++t) av[t][u] = *reinterpret_cast<const v4i*>(pa[t] + (c + u) * 32);
      xv[u] = *reinterpret_cast<const v4i*>(px + (c + u) * 32);
    }
  };
  auto mma = [&](const v4i (&av)[TR][kU], const v4i (&xv)[kU]) {
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int t = 0; t < TR; ++t)
        acc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[t][u], xv[u], acc[t], 0, 0, 0);
  };
  if (nsteps > 0) load(a0, x0, 0);
  int64_t st = 0;
  for (; st + 2 <= nsteps; st += 2) {
    load(a1, x1, (st + 1) * kU);
    mma(a0, x0);
    if (st + 2 < nsteps) load(a0, x0, (st + 2) * kU);
    mma(a1, x1);
  }
  if (st < nsteps) mma(a0, x0);
  for (int64_t c = nsteps * kU; c < nc; ++c) {
    const v4i x = *reinterpret_cast<const v4i*>(px + c * 32);
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      const v4i a = *reinterpret_cast<const v4i*>(pa[t] + c * 32);
      acc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, x, acc[t], 0, 0, 0);
    }
  }
#pragma unroll
  for (int t = 0; t < TR; ++t)
    store_tile(acc[t], lane, row0 + 32 * t, m, nrhs, E.mod[l], E.inv[l], res + l * res_stride);
}

// ------------------------------------------------------------------ on the fly
// grid ceil(m / 128); 8 waves, each 16 rows and the moduli l0 .. l0+NR-1 against CT tiles
// of 16 right-hand sides (v_mfma_i32_16x16x32_i8: NR x CT accumulators of 4 AGPRs, so the
// kernel fits two waves per SIMD).  Per K step of 32: lane (row = lane & 15, quarter
// kq = lane >> 4) loads the 8 fp64 values K = 32 c + 8 kq .. +7 of its row, scales and
// rounds them (row exponent from exps), turns them into 8 residue bytes per modulus and
// issues one MFMA per modulus and column tile against the X residues staged in LDS.  The
// next step's X residues are loaded into registers before this step's arithmetic and go
// to LDS after it.  A is loaded kPF steps ahead into a ring of registers.  When the rows
// are 16-byte aligned and k is a multiple of 32 (every K step below k is whole), every
// load of the loop is issued unconditionally from addresses clamped into A and X, in one
// fixed order per step, so the compiler's waits count exactly the loads a step needs;
// steps past k and rows holding Inf/NaN feed zeros.  Otherwise the loads are guarded and
// the waits drain every load in flight (same results, slower).
//
// Operand layout of the 16 x 16 x 32 instruction: lane supplies K = 8 (lane >> 4) .. +7 of
// row (A) or column (B) lane & 15; the accumulator holds rows 4 (lane >> 4) .. +3 of
// column lane & 15.
typedef long v1l;
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
// Moduli and their residue constants at compile time (the kernel is instantiated per pass
// of moduli L0 .. L0+NR-1), so no constant is loaded inside the loop.
constexpr RnsTable kRns = make_rns_table();

template <int L, int N, typename F>
__device__ __forceinline__ void for_moduli(F&& f) {
  if constexpr (L < N) {
    f(std::integral_constant<int, L>{});
    for_moduli<L + 1, N>(f);
  }
}

constexpr int kFlyWaves = 8;
constexpr int kFlyThreads = 64 * kFlyWaves;
constexpr int kFlyRows = 16 * kFlyWaves;     // rows per workgroup
// Staged X residues: per buffer and modulus, four planes (one per K quarter kq) of 32
// columns x 8 bytes, 288 bytes apart.  A fragment read (16 lanes of one kq, 16 columns)
// is 128 contiguous bytes; the two 8-byte halves a thread writes land in planes 2h and
// 2h + 1, whose 32-byte pad puts the writes of the two halves of 8 columns on disjoint
// banks.
constexpr int kXsPlane = 288;

template <bool kWide, int L0, int NR, int CT, bool kFast>
__global__ __launch_bounds__(kFlyThreads, 1) void gemv_fly_kernel(
    const double* __restrict__ a, int64_t m, int64_t k, int64_t lda,
    const int32_t* __restrict__ exps, const int8_t* __restrict__ xp, int64_t ldp,
    int64_t x_stride, int nrhs, int8_t* __restrict__ res, int64_t res_stride, int vec) {
  constexpr int l0 = L0;
  constexpr int kPF = !kFast ? 2 : NR * CT >= 30 ? 3 : 4;   // A steps in flight (registers)
  __shared__ __attribute__((aligned(16))) int8_t xs[2][NR][4][kXsPlane];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * kFlyWaves + (tid >> 6)) * 16;
  int64_t row = row0 + (lane & 15);
  row = row < m ? row : m - 1;
  const int kq = lane >> 4;
  int e = exps[row];
  const bool bad = e == INT32_MIN;
  if (bad) e = 0;
  const int64_t klim = bad ? 0 : k;  // a row with Inf/NaN contributes residues 0
  const double* pa = a + row * lda;

  v4i acc[NR][CT];
#pragma unroll
  for (int q = 0; q < NR; ++q)
#pragma unroll
    for (int t = 0; t < CT; ++t) acc[q][t] = v4i{0, 0, 0, 0};

  const int64_t nc = ldp / 32;
  const int64_t nc_k = (k + 31) / 32;   // K steps holding elements of A
  const bool any_bad = __ballot(bad) != 0;
  // X staging: NR moduli x 32 columns x 32 bytes = NR * 64 chunks of 16 bytes.
  constexpr int kXL = (NR * 64 + kFlyThreads - 1) / kFlyThreads;   // chunks per thread
  // Every thread loads its chunks (indexes past the last chunk re-read it); only the
  // owners store them.
  auto fetch_x = [&](v4i (&xr)[kXL], int64_t c) {
#pragma unroll
    for (int u = 0; u < kXL; ++u) {
      int idx = tid + kFlyThreads * u;
      idx = idx < NR * 64 ? idx : NR * 64 - 1;
      const int q = idx >> 6;
      int col = (idx >> 1) & 31;
      col = col < nrhs ? col : nrhs - 1;
      xr[u] = *reinterpret_cast<const v4i*>(xp + (int64_t)(l0 + q) * x_stride + col * ldp +
                                            c * 32 + 16 * (idx & 1));
    }
  };
  auto store_x = [&](const v4i(&xr)[kXL], int buf) {
#pragma unroll
    for (int u = 0; u < kXL; ++u) {
      const int idx = tid + kFlyThreads * u;
      if (idx < NR * 64) {
        const int q = idx >> 6, col = (idx >> 1) & 31, h = idx & 1;
        *reinterpret_cast<v1l*>(&xs[buf][q][2 * h][8 * col]) =
            (v1l)(((uint64_t)(uint32_t)xr[u][1] << 32) | (uint32_t)xr[u][0]);
        *reinterpret_cast<v1l*>(&xs[buf][q][2 * h + 1][8 * col]) =
            (v1l)(((uint64_t)(uint32_t)xr[u][3] << 32) | (uint32_t)xr[u][2]);
      }
    }
  };
  // Fast path: step c clamped into the steps below k, no condition per lane.
  auto load_a_fast = [&](double (&v)[8], int64_t c) {
    const int64_t h0 = (c < nc_k ? c : nc_k - 1) * 32 + 8 * kq;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const double2 d = *reinterpret_cast<const double2*>(pa + h0 + 2 * u);
      v[2 * u] = d.x;
      v[2 * u + 1] = d.y;
    }
  };
  auto load_a = [&](double (&v)[8], int64_t c) {
    const int64_t h0 = c * 32 + 8 * kq;
    if (vec && h0 + 8 <= klim) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const double2 d = *reinterpret_cast<const double2*>(pa + h0 + 2 * u);
        v[2 * u] = d.x;
        v[2 * u + 1] = d.y;
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = h0 + u < klim ? pa[h0 + u] : 0.0;
    }
  };

  v4i xr[kXL];
  // A ring of kPF steps: step c lives in va[c % kPF]; each step issues its X loads for step
  // c + 1 first, then its arithmetic, then A's loads for step c + kPF.  kFast (chosen by the
  // host): rows 16-byte aligned and k a multiple of 32.
  {
    double va[kPF][8];
#pragma unroll
    for (int i = 0; i < kPF; ++i) {
      if (kFast)
        load_a_fast(va[i], i);
      else
        load_a(va[i], i);
    }
    fetch_x(xr, 0);
    store_x(xr, 0);
    __syncthreads();
    const int64_t ncr = (nc + kPF - 1) / kPF * kPF;
    for (int64_t c0 = 0; c0 < ncr; c0 += kPF) {
#pragma unroll
      for (int ii = 0; ii < kPF; ++ii) {
        const int64_t c = c0 + ii;
        double(&cur)[8] = va[ii];
        const int buf = (int)(c & 1);
        if (c + 1 < nc) fetch_x(xr, c + 1);
        if (c < nc) {
          Prepared p[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            p[u] = prepare_element<kWide>(
                kFast && (c >= nc_k || (any_bad && bad)) ? 0.0 : cur[u], e);
          // Narrow residues two elements at a time: the low 16 bits of a' (the same for every
          // modulus) and of q = round(a' / m) of elements 2i, 2i+1 side by side, then one packed
          // 16-bit multiply-add q (-m) + a' gives both residues modulo 2^16 (their low bytes are
          // the residue bytes, as in residue_byte).
          uint32_t vpair[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vpair[i] = __builtin_amdgcn_perm(lo32(p[2 * i + 1].vm), lo32(p[2 * i].vm), 0x05040100u);
          for_moduli<0, NR>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            constexpr int l = l0 + q;
            uint32_t w0, w1;
            if constexpr (l == 0) {
              w0 = pack4(residue_byte_256(p[0]), residue_byte_256(p[1]), residue_byte_256(p[2]),
                         residue_byte_256(p[3]));
              w1 = pack4(residue_byte_256(p[4]), residue_byte_256(p[5]), residue_byte_256(p[6]),
                         residue_byte_256(p[7]));
            } else if constexpr (!kWide) {
              constexpr double inv = kRns.inv[l];
              constexpr uint16_t neg_m = (uint16_t)(0x10000 - kRns.moduli[l]);
              constexpr double kMagicD = 6755399441055744.0;
              uint32_t r2[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint32_t qa = lo32(__builtin_fma(p[2 * i].v, inv, kMagicD));
                const uint32_t qb = lo32(__builtin_fma(p[2 * i + 1].v, inv, kMagicD));
                const u16x2 qp =
                  __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(qb, qa, 0x05040100u));
                const u16x2 vp = __builtin_bit_cast(u16x2, vpair[i]);
                r2[i] = __builtin_bit_cast(uint32_t, qp * u16x2{neg_m, neg_m} + vp);
              }
              w0 = __builtin_amdgcn_perm(r2[1], r2[0], 0x06040200u);
              w1 = __builtin_amdgcn_perm(r2[3], r2[2], 0x06040200u);
            } else {
              constexpr double md = (double)kRns.moduli[l], inv = kRns.inv[l], c32 = kRns.c32[l];
              auto rb = [&](int u) { return residue_byte<kWide>(p[u], md, inv, c32); };
              w0 = pack4(rb(0), rb(1), rb(2), rb(3));
              w1 = pack4(rb(4), rb(5), rb(6), rb(7));
            }
            const v1l frag = (v1l)(((uint64_t)w1 << 32) | w0);
#pragma unroll
            for (int t = 0; t < CT; ++t) {
              const v1l xf =
                  *reinterpret_cast<const v1l*>(&xs[buf][q][kq][8 * (16 * t + (lane & 15))]);
              acc[q][t] = __builtin_amdgcn_mfma_i32_16x16x32_i8(frag, xf, acc[q][t], 0, 0, 0);
            }
          });
        }
        if (kFast)
          load_a_fast(cur, c + kPF);
        else
          load_a(cur, c + kPF);
        if (c + 1 < nc) store_x(xr, buf ^ 1);  // buffer buf ^ 1 was last read before the barrier
        __syncthreads();
      }
    }
  }
  if (row0 >= m) return;
#pragma unroll
  for (int q = 0; q < NR; ++q) {
    const int mod = kRns.moduli[l0 + q];
    const double inv = kRns.inv[l0 + q];
    int8_t* out = res + (int64_t)(l0 + q) * res_stride;
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      const int col = 16 * t + (lane & 15);
      if (col >= nrhs) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t rr = row0 + 4 * kq + v;
        if (rr < m) out[rr * nrhs + col] = (int8_t)sym_residue32(acc[q][t][v], mod, inv);
      }
    }
  }
}

GemvModuli gemv_moduli(int r) {
  GemvModuli E;
  const CrtConsts* C = crt_consts(r);
  for (int i = 0; i < kMaxModuli; ++i) {
    E.mod[i] = i < r ? C->mod[i] : 1;
    E.inv[i] = i < r ? C->inv[i] : 1.0;
  }
  return E;
}

template <bool kWide, int L0, int NR, int CT>
void launch_fly_ct(dim3 grid, hipStream_t s, const double* a, int64_t m, int64_t k, int64_t lda,
                   const int32_t* exps, const int8_t* xp, int64_t ldp, int64_t x_stride, int nrhs,
                   int8_t* res, int64_t res_stride) {
  const int vec = (reinterpret_cast<uintptr_t>(a) & 15) == 0 && (lda & 1) == 0;
  if (vec && k % 32 == 0 && k > 0)
    hipLaunchKernelGGL((gemv_fly_kernel<kWide, L0, NR, CT, true>), grid, dim3(kFlyThreads), 0, s,
                       a, m, k, lda, exps, xp, ldp, x_stride, nrhs, res, res_stride, vec);
  else
    hipLaunchKernelGGL((gemv_fly_kernel<kWide, L0, NR, CT, false>), grid, dim3(kFlyThreads), 0, s,
                       a, m, k, lda, exps, xp, ldp, x_stride, nrhs, res, res_stride, vec);
}

template <bool kWide, int L0, int NR>
void launch_fly(dim3 grid, hipStream_t s, const double* a, int64_t m, int64_t k, int64_t lda,
                const int32_t* exps, const int8_t* xp, int64_t ldp, int64_t x_stride, int nrhs,
                int8_t* res, int64_t res_stride) {
  if (nrhs <= 16)
    launch_fly_ct<kWide, L0, NR, 1>(grid, s, a, m, k, lda, exps, xp, ldp, x_stride, nrhs, res,
                                    res_stride);
  else
    launch_fly_ct<kWide, L0, NR, 2>(grid, s, a, m, k, lda, exps, xp, ldp, x_stride, nrhs, res,
                                    res_stride);
}

// Passes of moduli: 0 .. min(r, 16) - 1, then 16 .. r - 1.
template <bool kWide, int L0, int NR, int NMax>
void dispatch_fly(int nr, dim3 grid, hipStream_t s, const double* a, int64_t m, int64_t k,
                  int64_t lda, const int32_t* exps, const int8_t* xp, int64_t ldp,
                  int64_t x_stride, int nrhs, int8_t* res, int64_t res_stride) {
  if constexpr (NR <= NMax) {
    if (nr == NR)
      launch_fly<kWide, L0, NR>(grid, s, a, m, k, lda, exps, xp, ldp, x_stride, nrhs, res,
                                res_stride);
    else
      dispatch_fly<kWide, L0, NR + 1, NMax>(nr, grid, s, a, m, k, lda, exps, xp, ldp, x_stride,
                                            nrhs, res, res_stride);
  }
}

}  // namespace

int launch_gemv_stored(int64_t m, int64_t kp, int r, const int8_t* ap, int64_t lda_p,
                       int64_t a_stride, const int8_t* xp, int64_t x_stride, int nrhs,
                       int8_t* res, hipStream_t s) {
  if (m <= 0) return OZK_OK;
  // Two row tiles per wave: every X fragment (an L2 read) feeds two MFMAs; measured
  // faster than one or four tiles for 1, 8 and 32 right-hand sides at 32768 x 32768.
  constexpr int kTr = 2;
  dim3 grid((unsigned)((m + 128 * kTr - 1) / (128 * kTr)), (unsigned)r);
  hipLaunchKernelGGL(gemv_stored_kernel<kTr>, grid, dim3(256), 0, s, ap, lda_p, a_stride, m, xp,
                     kp, x_stride, nrhs, res, m * nrhs, gemv_moduli(r));
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

int launch_gemv_fly(const double* a, int64_t m, int64_t k, int64_t lda, const int32_t* exps,
                    int r, int p_bits, const int8_t* xp, int64_t ldp, int64_t x_stride, int nrhs,
                    int8_t* res, hipStream_t s) {
  if (m <= 0) return OZK_OK;
  if (!residue_consts(r, p_bits)) return OZK_EINVAL;
  const bool wide = residue_consts(r, p_bits)->wide;
  dim3 grid((unsigned)((m + kFlyRows - 1) / kFlyRows));
  // At most 16 moduli per pass (16 x 2 accumulator tiles = 128 registers); r > 16 takes two.
  const int n0 = r < 16 ? r : 16;
  if (wide)
    dispatch_fly<true, 0, 1, 16>(n0, grid, s, a, m, k, lda, exps, xp, ldp, x_stride, nrhs, res,
                                 m * nrhs);
  else
    dispatch_fly<false, 0, 1, 16>(n0, grid, s, a, m, k, lda, exps, xp, ldp, x_stride, nrhs, res,
                                  m * nrhs);
  if (hipGetLastError() != hipSuccess) return OZK_EHIP;
  if (r > 16) {
    if (wide)
      dispatch_fly<true, 16, 1, kMaxModuli - 16>(r - 16, grid, s, a, m, k, lda, exps, xp, ldp,
                                                 x_stride, nrhs, res, m * nrhs);
    else
      dispatch_fly<false, 16, 1, kMaxModuli - 16>(r - 16, grid, s, a, m, k, lda, exps, xp, ldp,
                                                  x_stride, nrhs, res, m * nrhs);
    if (hipGetLastError() != hipSuccess) return OZK_EHIP;
  }
  return OZK_OK;
}

}  // namespace ozk
