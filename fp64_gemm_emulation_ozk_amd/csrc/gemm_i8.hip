// Exact int8 x int8 -> int32 matrix products, one per modulus, on the gfx950 MFMA
// units (v_mfma_i32_32x32x32_i8).  [TME4] abstract: the tensor term of Ozaki scheme II;
// [AWE] abstract: each product is an error-free integer matrix product.
//
// Operands are residue planes with K contiguous: A_l [m][kp], B_l [n][kp] (B already
// transposed by the deconstruction), kp a multiple of 64 and zero-padded, so the K loop
// has no tail.  |residue| <= 128 and kp <= 131072 keep every int32 sum exact.
//
// Tiling: workgroup tile 256 x 256 x 64, 256 threads = 4 waves, each wave a 128 x 128
// block of 4 x 4 MFMA tiles of 32 x 32 (256 accumulator registers, held in AGPRs), so
// every 16-byte LDS fragment read feeds two MFMAs.  Global tiles go through two sets of
// registers into double-buffered LDS (64 KiB), with the MFMA, LDS and global-memory
// instructions of each K sub-step interleaved explicitly (see the pipeline below); LDS rows are 64 bytes with the four 16-byte chunks
// XOR-swizzled by (row >> 1) & 3 so that the fragment reads of 8 consecutive rows hit 8
// distinct bank groups.  Workgroups are mapped XCD by XCD (the hardware deals them out
// round-robin over the 8 XCDs) onto contiguous runs of tiles, ordered in groups of 4
// tile rows, so the tiles in flight on one XCD share A rows and B columns in its L2.
//
// Epilogues: the int32 products themselves, or their symmetric residues modulo m_l as
// int8 (what the CRT reconstruction consumes: 1 byte instead of 4 per output).
#include <type_traits>

#include "ozk_internal.h"

namespace ozk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;
constexpr int kThreads = 256;
constexpr int kLdsA = BM * BK;   // bytes per stage
constexpr int kLdsB = BN * BK;

struct EpiModuli {
  int32_t mod[kMaxModuli];
  double inv[kMaxModuli];
};

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ ((row >> 1) & 3)) << 4);
}

// Symmetric residue of an exact int32 product modulo m (m odd <= 255, or 256).
__device__ __forceinline__ int sym_residue(int v, int m, double inv) {
  if (m == 256) return (int)(int8_t)(v & 0xff);
  constexpr double kMagicD = 6755399441055744.0;
  double d = (double)v;
  double q = __builtin_fma(d, inv, kMagicD) - kMagicD;
  return (int)__builtin_fma(-q, (double)m, d);
}

template <int kEpi>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_kernel(
    int64_t m, int64_t n, int64_t kp, const int8_t* __restrict__ pa, int64_t stride_a,
    const int8_t* __restrict__ pb, int64_t stride_b, void* __restrict__ out, int64_t ldo,
    int64_t stride_o, int tiles_m, int tiles_n, EpiModuli E) {
  __shared__ __attribute__((aligned(16))) int8_t lds[2 * (kLdsA + kLdsB)];

  // Block -> (modulus, tile row, tile column): XCD-contiguous, then grouped by kGroupM.
  const int total = gridDim.x;
  int bid = blockIdx.x;
  if (total % kXcds == 0) bid = (bid % kXcds) * (total / kXcds) + bid / kXcds;
  const int per_mod = tiles_m * tiles_n;
  const int l = bid / per_mod;
  const int rem = bid - l * per_mod;
  const int per_group = kGroupM * tiles_n;
  const int first_m = (rem / per_group) * kGroupM;
  const int gsize = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  const int in_group = rem % per_group;
  const int tm = first_m + in_group % gsize;
  const int tn = in_group / gsize;

  const int8_t* A = pa + l * stride_a;
  const int8_t* B = pb + l * stride_b;
  const int64_t row0 = (int64_t)tm * BM;
  const int64_t col0 = (int64_t)tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1;   // 0..1: rows wr*128
  const int wc = wave & 1;    // 0..1: cols wc*128

  // Global load assignment: 16-byte chunk q = tid + 256*s, row q >> 2, chunk q & 3.
  const int64_t last_a = m - 1, last_b = n - 1;
  const int8_t* ga[4];
  int sa[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    int q = tid + kThreads * s;
    int r = q >> 2, c = q & 3;
    int64_t gr = row0 + r;
    gr = gr < last_a ? gr : last_a;
    ga[s] = A + gr * kp + c * 16;
    sa[s] = swz(r, c);
  }
  const int8_t* gb[4];
  int sb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    int q = tid + kThreads * s;
    int r = q >> 2, c = q & 3;
    int64_t gr = col0 + r;
    gr = gr < last_b ? gr : last_b;
    gb[s] = B + gr * kp + c * 16;
    sb[s] = swz(r, c);
  }

  v16i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  // Software pipeline over K tiles of 64 (two MFMA sub-steps of K = 32 each):
  //   sub-step 0 of tile t: 16 MFMAs on fragments (t, 0), interleaved with the global
  //     loads of tile t+2 into register set t%2, the LDS writes of tile t+1 (register
  //     set (t+1)%2, loaded one tile earlier) and the fragment reads of (t, 1);
  //   sub-step 1 of tile t: barrier (tile t+1 visible), then 16 MFMAs on (t, 1)
  //     interleaved with the fragment reads of (t+1, 0).
  // Loads past the last tile are clamped to it (in bounds, results unused), so each
  // sub-step is a single basic block that the scheduling groups below can interleave.
  v4i ra[2][4], rb[2][4];   // global tiles in flight
  v4i fa[2][4], fb[2][4];   // MFMA fragments of the current and next sub-step
  const int64_t nk = kp / BK;
  auto load_global = [&](v4i (&xa)[4], v4i (&xb)[4], int64_t t) {
    const int64_t k0 = (t < nk ? t : nk - 1) * BK;
#pragma unroll
    for (int s = 0; s < 4; ++s) xa[s] = *reinterpret_cast<const v4i*>(ga[s] + k0);
#pragma unroll
    for (int s = 0; s < 4; ++s) xb[s] = *reinterpret_cast<const v4i*>(gb[s] + k0);
  };
  auto store_lds = [&](int buf, const v4i (&xa)[4], const v4i (&xb)[4]) {
    int8_t* la = lds + buf * (kLdsA + kLdsB);
    int8_t* lb = la + kLdsA;
#pragma unroll
    for (int s = 0; s < 4; ++s) *reinterpret_cast<v4i*>(la + sa[s]) = xa[s];
#pragma unroll
    for (int s = 0; s < 4; ++s) *reinterpret_cast<v4i*>(lb + sb[s]) = xb[s];
  };
  // Fragment reads: lane holds row (lane & 31) of a 32-row block and 16 bytes at
  // K offset 32*kk + 16*(lane >> 5); A and B use the same K map, so the product is
  // independent of how the instruction orders K internally.
  const int frow = lane & 31;
  const int fchunk = lane >> 5;
  auto read_frags = [&](v4i (&xa)[4], v4i (&xb)[4], int buf, int kk) {
    const int8_t* la = lds + buf * (kLdsA + kLdsB);
    const int8_t* lb = la + kLdsA;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      xa[i] = *reinterpret_cast<const v4i*>(la + swz(wr * 128 + i * 32 + frow, kk * 2 + fchunk));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      xb[j] = *reinterpret_cast<const v4i*>(lb + swz(wc * 128 + j * 32 + frow, kk * 2 + fchunk));
  };
  auto mfma16 = [&](const v4i (&xa)[4], const v4i (&xb)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa[i], xb[j], acc[i][j], 0, 0, 0);
  };

  load_global(ra[0], rb[0], 0);
  load_global(ra[1], rb[1], 1);
  store_lds(0, ra[0], rb[0]);
  __syncthreads();
  read_frags(fa[0], fb[0], 0, 0);

  auto tile_step = [&](auto parity, int64_t t) {
    constexpr int p = decltype(parity)::value;
    // sub-step 0
    __builtin_amdgcn_sched_barrier(0);
    load_global(ra[p], rb[p], t + 2);
    store_lds(p ^ 1, ra[p ^ 1], rb[p ^ 1]);
    read_frags(fa[1], fb[1], p, 1);
    mfma16(fa[0], fb[0]);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
    }
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 1
    __syncthreads();
    read_frags(fa[0], fb[0], p ^ 1, 0);
    mfma16(fa[1], fb[1]);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  int64_t t = 0;
  for (; t + 2 <= nk; t += 2) {
    tile_step(std::integral_constant<int, 0>(), t);
    tile_step(std::integral_constant<int, 1>(), t + 1);
  }
  if (t < nk) tile_step(std::integral_constant<int, 0>(), t);

  // Output layout of a 32x32 MFMA tile: lane -> column (lane & 31); register v ->
  // row 8*(v/4) + 4*(lane/32) + (v%4).
  const int mod = E.mod[l];
  const double inv = E.inv[l];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = col0 + wc * 128 + j * 32 + (lane & 31);
      if (col >= n) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = row0 + wr * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row >= m) continue;
        const int64_t off = l * stride_o + row * ldo + col;
        if (kEpi == kEpiProducts)
          reinterpret_cast<int32_t*>(out)[off] = acc[i][j][v];
        else
          reinterpret_cast<int8_t*>(out)[off] = (int8_t)sym_residue(acc[i][j][v], mod, inv);
      }
    }
  }
}

}  // namespace

int launch_gemm_i8(int64_t m, int64_t n, int64_t kp, int r, const int8_t* pa, int64_t stride_a,
                   const int8_t* pb, int64_t stride_b, void* out, int64_t ldo, int64_t stride_o,
                   int epilogue, hipStream_t s) {
  if (m <= 0 || n <= 0) return OZK_OK;
  const int tiles_m = (int)((m + BM - 1) / BM);
  const int tiles_n = (int)((n + BN - 1) / BN);
  EpiModuli E;
  const CrtConsts* C = crt_consts(r);
  for (int i = 0; i < kMaxModuli; ++i) {
    E.mod[i] = i < r ? C->mod[i] : 1;
    E.inv[i] = i < r ? C->inv[i] : 1.0;
  }
  const int64_t blocks = (int64_t)tiles_m * tiles_n * r;
  if (blocks > 0x7fffffff) return OZK_EUNSUPPORTED;
  if (epilogue == kEpiProducts)
    hipLaunchKernelGGL(gemm_i8_kernel<kEpiProducts>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       s, m, n, kp, pa, stride_a, pb, stride_b, out, ldo, stride_o, tiles_m,
                       tiles_n, E);
  else
    hipLaunchKernelGGL(gemm_i8_kernel<kEpiResidues>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       s, m, n, kp, pa, stride_a, pb, stride_b, out, ldo, stride_o, tiles_m,
                       tiles_n, E);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

}  // namespace ozk
