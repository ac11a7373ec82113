// Exact int8 x int8 -> int32 matrix products, one per modulus, on the gfx950 MFMA
// units (v_mfma_i32_16x16x64_i8 in the persistent kernel, v_mfma_i32_32x32x32_i8 in the
// one-tile-per-workgroup kernel).  [TME4] abstract: the tensor term of Ozaki scheme II;
// [AWE] abstract: each product is an error-free integer matrix product.
//
// Operands are residue planes with K contiguous: A_l [m][kp], B_l [n][kp] (B already
// transposed by the deconstruction), kp a multiple of 64 and zero-padded, so the K loop
// has no tail.  |residue| <= 128 and kp <= 131072 keep every int32 sum exact.
//
// Two kernels share the workgroup tiling below: gemm_i8_pairs_kernel (K in steps of 128,
// at least two of them: persistent, whole-cache-line loads, 16 x 16 x 64 MFMAs, described
// above it) and gemm_i8_kernel (any K that is a multiple of 64: one workgroup per tile,
// 32 x 32 x 32 MFMAs, described here).
//
// Tiling: workgroup tile 256 x 256 x 64, 512 threads = 8 waves, two per SIMD.  Waves
// 0..3 own rows 0..127 of the tile, waves 4..7 rows 128..255; each wave a 128 x 64 block
// of 4 x 2 MFMA tiles of 32 x 32 (128 accumulator registers).  Each K step is two halves
// of 8 MFMAs around one workgroup barrier; the fragments of the next half are read from
// LDS between the MFMAs of the current one, and the two waves of a SIMD cover each
// other's waits.  Global tiles go straight into a 5-deep LDS ring (32 KiB per K step) by
// global_load_lds_dwordx4, issued between MFMAs from a wave-uniform SGPR base plus a
// fixed per-lane offset into the stage consumed one barrier earlier, five K steps ahead.
// LDS rows are 64 bytes with the four 16-byte chunks XOR-swizzled by (row >> 2) & 3, so
// the 16 lanes of a fragment read (16 consecutive rows, one chunk each) cover all 64
// banks.  Workgroups are mapped XCD by XCD (the hardware deals them out round-robin over
// the 8 XCDs) onto contiguous runs of tiles, ordered in groups of 4 tile rows, so the
// tiles in flight on one XCD share A rows and B columns in its L2.
//
// Epilogues: the int32 products themselves, or their symmetric residues modulo m_l as
// int8 (what the CRT reconstruction consumes: 1 byte instead of 4 per output), staged
// through LDS as one 256 x 256 byte tile so that every global store writes 256-byte rows.
#include <atomic>
#include <type_traits>

#include <hip/hip_ext.h>

#include "lds_dma.h"
#include "ozk_internal.h"

namespace ozk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;
constexpr int kWavesDefault = 8;  // waves per workgroup of the launched kernel
constexpr int kLdsA = BM * BK;   // bytes per stage
constexpr int kLdsB = BN * BK;

struct EpiModuli {
  int32_t mod[kMaxModuli];
  double inv[kMaxModuli];
};

// gfx950 LDS serves a 16-byte-per-lane read 16 lanes at a time from 64 four-byte banks
// (256 bytes per clock): lanes 0..15 of a fragment read rows r..r+15 at the same logical
// chunk, and rows with equal (row mod 4) would hit the same banks without the XOR.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ ((row >> 2) & 3)) << 4);
}

// Low byte of the symmetric residue of an exact int32 product v modulo an odd m <= 255.
// q = round(v / m) is read from the low word of v * RN(1/m) + 1.5 * 2^52: the product is
// within 2^-30 of v / m, whose distance to a half-integer is at least 1 / (2m), so the
// rounding is exact.  The residue v - q m lies in [-(m-1)/2, (m-1)/2]; its low byte is
// (v - q m) mod 2^8, for which the low 24 bits of q suffice: one signed 24-bit
// multiply-add q * (-m) + v (v_mad_i32_i24).
__device__ __forceinline__ uint32_t residue_byte_odd(int v, uint32_t m, double inv) {
  constexpr double kMagicD = 6755399441055744.0;
  const double t = __builtin_fma((double)v, inv, kMagicD);
  const int q = (int)(uint32_t)__double_as_longlong(t);
  return (uint32_t)(__mul24(q, -(int)m) + v);
}

// Bytes 0 of four words into one word (b0 lowest).
__device__ __forceinline__ uint32_t pack4b(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Workgroup barrier that is also a compiler barrier for memory operations, so that no
// LDS access is moved across it.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr int kStages = 5;                    // LDS ring of K steps: 160 KiB
constexpr int kStageBytes = kLdsA + kLdsB;    // 32 KiB: A rows 0..255 then B rows 0..255
constexpr int kOutPitch = BN + 8;  // residue staging: 2 rows apart = 1 bank apart (dwords)

// Wave layout of a 256 x 256 tile: NW waves in 2 rows x NW/2 columns, each wave WM x WN
// = 128 x (512 / NW) outputs as TI x TJ MFMA blocks of 32 x 32.
template <int NW>
struct WaveLayout {
  static constexpr int kThreads = 64 * NW;
  static constexpr int WN = 2 * BN / NW;
  static constexpr int TI = 4, TJ = WN / 32;
  static constexpr int kLoads = kStageBytes / 1024 / NW;  // 1 KiB load instructions per step
  static constexpr int kMfmaHalf = TI * TJ;
  static_assert(kMfmaHalf >= TI + TJ && kMfmaHalf == 2 * kLoads, "load and read slots");
};
static_assert(BM * kOutPitch <= kStages * kStageBytes, "residue staging must fit the ring");

// Epilogue of a 256 x 256 tile: the int32 products, or their residues modulo m_l staged
// through LDS (the ring is free: every wave has passed its last read and load wait).
template <int kEpi, int NW>
__device__ __forceinline__ void tile_epilogue(
    const v16i (&acc)[WaveLayout<NW>::TI][WaveLayout<NW>::TJ], int8_t* lds, int64_t m,
    int64_t n, int l, int64_t row0, int64_t col0, int grp, int wq, int wave, int lane,
    const EpiModuli& E, void* __restrict__ out, int64_t ldo, int64_t stride_o, int vec_out) {
  using WL = WaveLayout<NW>;
  constexpr int TI = WL::TI, TJ = WL::TJ;

  // The MFMA runs with the B fragment as its first operand, so each accumulator tile is
  // C^T: lane -> row (lane & 31) of the 32 x 32 block of C, register v -> column
  // 8*(v/4) + 4*(lane/32) + (v%4); registers 4q..4q+3 hold 4 consecutive columns.
  const int mod = E.mod[l];
  const double inv = E.inv[l];
  const int64_t wrow0 = row0 + grp * 128, wcol0 = col0 + wq * WL::WN;
  if (kEpi == kEpiProducts) {
    int32_t* o = reinterpret_cast<int32_t*>(out) + l * stride_o;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int64_t row = wrow0 + i * 32 + (lane & 31);
      if (row >= m) continue;
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t col = wcol0 + j * 32 + 8 * q + 4 * (lane >> 5);
          int32_t* dst = o + row * ldo + col;
          if (vec_out && col + 4 <= n) {
            *reinterpret_cast<v4i*>(dst) = v4i{acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                               acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (col + u < n) dst[u] = acc[i][j][4 * q + u];
          }
        }
    }
    return;
  }
  // Residues: stage the 256 x 256 byte tile in LDS (row pitch 264: the dword writes of
  // 64 lanes hit distinct banks), then each wave stores 32 rows, 16 lanes x 16 bytes per
  // 256-byte row.
  wg_barrier();  // every wave is past its reads and loads of the ring
  int8_t* tile = lds;
  // m = 256 keeps the low byte of the product; odd moduli reduce (uniform branch, taken
  // once per tile rather than per element).
  auto stage = [&](auto byte_of) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w = pack4b(byte_of(acc[i][j][4 * q]), byte_of(acc[i][j][4 * q + 1]),
                                    byte_of(acc[i][j][4 * q + 2]), byte_of(acc[i][j][4 * q + 3]));
          *reinterpret_cast<uint32_t*>(tile + (grp * 128 + i * 32 + (lane & 31)) * kOutPitch +
                                       wq * WL::WN + j * 32 + 8 * q + 4 * (lane >> 5)) = w;
        }
  };
  if (mod == 256) {
    stage([](int v) { return (uint32_t)v; });
  } else {
    const uint32_t um = (uint32_t)mod;
    stage([=](int v) { return residue_byte_odd(v, um, inv); });
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  wg_barrier();  // the whole tile is staged
  int8_t* o = reinterpret_cast<int8_t*>(out) + l * stride_o;
#pragma unroll 4
  for (int s4 = 0; s4 < 64 / NW; ++s4) {
    const int rl = wave * (BM / NW) + s4 * 4 + (lane >> 4), cl = 16 * (lane & 15);
    const int64_t row = row0 + rl, col = col0 + cl;
    const int8_t* srcp = tile + rl * kOutPitch + cl;
    const uint2 lo = *reinterpret_cast<const uint2*>(srcp);
    const uint2 hi = *reinterpret_cast<const uint2*>(srcp + 8);
    if (row >= m) continue;
    int8_t* dst = o + row * ldo + col;
    if (vec_out && col + 16 <= n) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
      const uint32_t wv[4] = {lo.x, lo.y, hi.x, hi.y};
      for (int u = 0; u < 16; ++u)
        if (col + u < n) dst[u] = (int8_t)(wv[u >> 2] >> (8 * (u & 3)));
    }
  }
}


template <int kEpi, int NW>
__global__ __launch_bounds__(64 * NW, 1) void gemm_i8_kernel(
    int64_t m, int64_t n, int64_t kp, const int8_t* __restrict__ pa, int64_t stride_a,
    const int8_t* __restrict__ pb, int64_t stride_b, void* __restrict__ out, int64_t ldo,
    int64_t stride_o, int tiles_m, int tiles_n, EpiModuli E, int vec_out) {
  __shared__ __attribute__((aligned(1024))) int8_t lds[kStages * kStageBytes];

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

  using WL = WaveLayout<NW>;
  constexpr int TI = WL::TI, TJ = WL::TJ, kWaves = NW, kRegionsPerWave = WL::kLoads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = __builtin_amdgcn_readfirstlane(wave / (NW / 2));  // rows grp*128 (uniform)
  const int wq = __builtin_amdgcn_readfirstlane(wave % (NW / 2));   // columns wq*WN (uniform)

  // Direct-load sources: wave w fills regions w, w+8, w+16, w+24 of a stage; region rg
  // holds 16 rows of A (rg < 16) or B, 64 bytes each; lane i lands at row 16*(rg%16) + i/4,
  // physical chunk i%4, which holds logical K chunk (i%4) ^ ((row >> 2) & 3) (the
  // read-side swizzle).
  // Sources are addressed as a wave-uniform base (tile origin of A or B plus the K offset,
  // in SGPRs) plus a fixed 32-bit lane offset (row within the tile, clamped to the last
  // row of the matrix, times kp, plus the chunk); regions 0..15 are A, 16..31 B.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint64_t sbase_a = (uint64_t)(A + row0 * kp), sbase_b = (uint64_t)(B + col0 * kp);
  uint32_t voff[kRegionsPerWave];
#pragma unroll
  for (int q = 0; q < kRegionsPerWave; ++q) {
    const int rg = wave + kWaves * q;
    const bool is_b = rg >= 16;
    const int row = 16 * (rg & 15) + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    const int64_t origin = is_b ? col0 : row0;
    const int64_t last = (is_b ? n : m) - 1;
    const int64_t gr = origin + row < last ? origin + row : last;
    voff[q] = (uint32_t)((gr - origin) * kp + 16 * chunk);
  }
  auto region_base = [&](int q) {  // uniform: region wave + NW q is B iff it is >= 16
    return wave_u + kWaves * q >= 16 ? sbase_b : sbase_a;
  };
  const uint32_t lds0 = lds_address(lds);
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(lds0 + wave * 1024);
  const int nk = (int)(kp / BK);
  auto issue_step = [&](int t) {  // K step t (clamped to the last) into stage t % kStages
    const int tc = t < nk ? t : nk - 1;
    const uint32_t base = wave_lds + (uint32_t)(t % kStages) * kStageBytes;
#pragma unroll
    for (int q = 0; q < kRegionsPerWave; ++q)
      dma16_sbase(voff[q], region_base(q) + (uint64_t)tc * BK, base + q * (kWaves * 1024));
  };

  v16i acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  // Fragment reads: lane holds row (lane & 31) of a 32-row block and 16 bytes at
  // K offset 32*kk + 16*(lane >> 5); A and B use the same K map, so the product is
  // independent of how the instruction orders K internally.
  const int frow = lane & 31;
  const int fchunk = lane >> 5;
  int offa[TI], offb[TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i) offa[i] = (grp * 128 + i * 32 + frow) * BK;
#pragma unroll
  for (int j = 0; j < TJ; ++j) offb[j] = kLdsA + (wq * WL::WN + j * 32 + frow) * BK;
  const int sw = (frow >> 2) & 3;  // row swizzle (the same for every block: 32 | block rows)
  v4i fa[2][TI], fb[2][TJ];

  // Schedule: every wave runs the same two halves per K step, one barrier between them:
  //   half 0 of step t: the 8 MFMAs of K half 0, reading the K half 1 fragments of step t
  //   between them; then wait for this wave's loads of step t+1 and for its reads;
  //   barrier: step t+1 is complete in LDS and every wave has finished reading step t;
  //   half 1: the 8 MFMAs of K half 1, reading step t+1's K half 0 fragments and issuing
  //   this wave's 4 loads of step t+kStages into the stage of step t (just consumed).
  // Loads therefore run kStages - 1 full steps ahead of their wait; younger than the last
  // load of step t+1 at the wait are those of steps t+2 .. t+kStages-1.
#pragma unroll
  for (int t = 0; t < kStages; ++t) issue_step(t);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kRegionsPerWave * (kStages - 1)) : "memory");
  wg_barrier();
  {
    const int8_t* st = lds;
    const int c = (fchunk ^ sw) << 4;
#pragma unroll
    for (int i = 0; i < TI; ++i) fa[0][i] = *reinterpret_cast<const v4i*>(st + offa[i] + c);
#pragma unroll
    for (int j = 0; j < TJ; ++j) fb[0][j] = *reinterpret_cast<const v4i*>(st + offb[j] + c);
  }
  for (int t = 0; t < nk; ++t) {
    __builtin_amdgcn_sched_barrier(0);
    const int8_t* st = lds + (t % kStages) * kStageBytes;
    const int c1 = ((2 + fchunk) ^ sw) << 4;
#pragma unroll
    for (int idx = 0; idx < WL::kMfmaHalf; ++idx) {
      const int i = idx / TJ, j = idx % TJ;
      acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[0][j], fa[0][i], acc[i][j], 0, 0, 0);
      if (idx < TI)
        fa[1][idx] = *reinterpret_cast<const v4i*>(st + offa[idx] + c1);
      else if (idx < TI + TJ)
        fb[1][idx - TI] = *reinterpret_cast<const v4i*>(st + offb[idx - TI] + c1);
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kRegionsPerWave * (kStages - 2)) : "memory");
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    wg_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int tn = t + 1 < nk ? t + 1 : t;  // past the last step: a harmless re-read
    const int8_t* sn = lds + (tn % kStages) * kStageBytes;
    const int c0 = (fchunk ^ sw) << 4;
    const int tl = t + kStages;
    const int64_t koff = (int64_t)(tl < nk ? tl : nk - 1) * BK;
    const uint32_t lbase = wave_lds + (uint32_t)(t % kStages) * kStageBytes;
#pragma unroll
    for (int idx = 0; idx < WL::kMfmaHalf; ++idx) {
      const int i = idx / TJ, j = idx % TJ;
      acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[1][j], fa[1][i], acc[i][j], 0, 0, 0);
      if (idx < TI)
        fa[0][idx] = *reinterpret_cast<const v4i*>(sn + offa[idx] + c0);
      else if (idx < TI + TJ)
        fb[0][idx - TI] = *reinterpret_cast<const v4i*>(sn + offb[idx - TI] + c0);
      if ((idx & 1) == 1)
        dma16_sbase(voff[idx >> 1], region_base(idx >> 1) + (uint64_t)koff,
                    lbase + (idx >> 1) * (kWaves * 1024));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // The clamped loads past the last K step are still landing in the ring.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  tile_epilogue<kEpi, NW>(acc, lds, m, n, l, row0, col0, grp, wq, wave, lane, E, out, ldo,
                          stride_o, vec_out);
}


// Residues of one 256 x 256 tile stored straight from the accumulators (no LDS: the ring
// already holds the next tile's first K steps).  Lane (row lane & 31, half h = lane >> 5)
// of an MFMA block holds columns 8 q + 4 h .. +3 in registers 4 q .. 4 q + 3; after the
// bytes are packed one word per q, two v_permlane32_swap exchanges (words 0 <-> 2 and
// 1 <-> 3 across the halves) leave lane h with columns 16 h .. 16 h + 15 of its row, one
// 16-byte store.  A full tile issues exactly TI * TJ stores per wave.
template <int NW>
__device__ __forceinline__ void store_residues_direct(
    const v16i (&acc)[WaveLayout<NW>::TI][WaveLayout<NW>::TJ], int64_t m, int64_t n,
    int64_t row0, int64_t col0, int grp, int wq, int lane, int mod, double inv,
    int8_t* __restrict__ o, int64_t ldo, bool full, int vec_out) {
  using WL = WaveLayout<NW>;
  auto emit = [&](auto byte_of) {
#pragma unroll
    for (int i = 0; i < WL::TI; ++i)
#pragma unroll
      for (int j = 0; j < WL::TJ; ++j) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = pack4b(byte_of(acc[i][j][4 * q]), byte_of(acc[i][j][4 * q + 1]),
                        byte_of(acc[i][j][4 * q + 2]), byte_of(acc[i][j][4 * q + 3]));
        const auto s02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
        const uint4 v = make_uint4(s02[0], s02[1], s13[0], s13[1]);
        const int64_t row = row0 + grp * 128 + i * 32 + (lane & 31);
        const int64_t col = col0 + wq * WL::WN + j * 32 + 16 * (lane >> 5);
        int8_t* dst = o + row * ldo + col;
        if (full) {
          *reinterpret_cast<uint4*>(dst) = v;
        } else if (row < m) {
          if (vec_out && col + 16 <= n) {
            *reinterpret_cast<uint4*>(dst) = v;
          } else {
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
            for (int u = 0; u < 16; ++u)
              if (col + u < n) dst[u] = (int8_t)(wv[u >> 2] >> (8 * (u & 3)));
          }
        }
      }
  };
  if (mod == 256) {
    emit([](int v) { return (uint32_t)v; });
  } else {
    const uint32_t um = (uint32_t)mod;
    emit([=](int v) { return residue_byte_odd(v, um, inv); });
  }
}

// Pair-stage persistent variant for kp a multiple of 128 with at least two pairs: the LDS
// ring holds two stages of two K steps each (64 KiB: A rows 0..255, then B rows 0..255,
// 128 bytes per row), so every direct load moves 8 rows x 128 bytes (whole cache lines)
// instead of 16 rows x 64 bytes (half lines), which is what limits the L2 -> LDS stream of
// the 64-byte ring.  The eight 16-byte chunks of a row are XOR-swizzled by (row >> 1) & 7:
// the 16 lanes of a fragment read (rows r .. r+15, one logical chunk) then cover all 64
// banks.
//
// Every wave's 128 x 64 outputs are 8 x 4 blocks of 16 x 16 on v_mfma_i32_16x16x64_i8
// (32 accumulators of 4 registers; on random operands this shape sustains about 17 % more
// operations per second under the board's power limit than 32 x 32 x 32).  Per pair p
// (K bytes 128 p .. 128 p + 127) every wave runs four quarters of 16 MFMAs; quarter q
// covers row blocks 2q and 2q+1 against all four column blocks, and each block's two K
// halves go to the matrix core back to back, the second MFMA taking the first one's
// result as its accumulator (8192^3, r = 16: 6.753 -> 6.657 ms against the K-half-major
// order, bit-identical; a register-only loop of this shape issues 5 % more operations per
// second in that order).  A fragment is 16 rows x 64 K bytes (lane -> row lane % 16,
// 16-byte chunk lane / 16 of the K half; A and B the same); the wave holds all 8 B
// fragments of the pair and the 4 A fragments of one quarter, and reads the next
// quarter's A fragments during the first MFMAs of a quarter.  After quarter 2 the wave
// waits for its loads of pair p+1 and for its reads, and the workgroup barrier makes pair
// p+1 complete and pair p fully read; quarter 3 then reads pair p+1's A fragments of
// quarter 0, replaces each B fragment right after its last use in this pair, and issues
// all 8 of this wave's loads of pair p+2 into pair p's buffer (one after every second
// MFMA), so every load has three quarters to land before its wait.
//
// One workgroup per CU walks a fixed list of tiles.  Pair numbers run on across tiles:
// the last two pairs of a tile load the next tile's pairs 0 and 1 (both before the
// epilogue), and its last quarter reads the next tile's first fragments, so the epilogue
// (residues stored from registers) overlaps those loads, and the wait for pair 1 after
// the next tile's first three quarters lets the epilogue's stores stay in flight (vector
// memory operations count down in issue order, so vmcnt(number of stores) covers every
// load issued before them).
// Tile order and placement: the kernel runs under the board's power limit, so fewer bytes
// fetched from HBM per product is time saved.  The launch has G workgroups (one per CU,
// G a multiple of 8); round j is the G consecutive tiles G j .. G j + G - 1 of the order
// (modulus, groups of kPairGroupM = 8 tile rows, column, row in group), and the G / 8
// workgroups of one XCD (the hardware deals workgroups out round-robin over the 8 XCDs)
// take one contiguous run of it: 8 tile rows x 4 tile columns at the 8192 x 8192 shape,
// 12 panels of A and B for 32 tiles in that XCD's L2.  All XCDs work on the same modulus
// and the same 8 tile rows at once, so the A panels and (from one group of rows to the
// next) the B panels they share come from the 256 MB last-level cache rather than HBM.
constexpr int kPairRow = 128;                       // bytes per row of a pair stage
constexpr int kPairGroupM = 8;                      // tile rows per group of the tile order
constexpr int kPairBytes = (BM + BN) * kPairRow;    // 64 KiB

// Residues of one 256 x 256 tile stored straight from the 16 x 16 accumulators.  The MFMA
// runs with the B fragment first, so lane l of block (i, j) holds row 16 i + l % 16 and the
// four consecutive columns 16 j + 4 (l / 16) + 0..3 in its 4 registers (one word once
// packed to bytes).  For one row block the four lanes l % 16 + {0, 16, 32, 48} hold a
// 4 x 4 matrix of words M[lane group][j]; a v_permlane32_swap and a v_permlane16_swap on
// each of two word pairs transpose it, leaving lane group g with M[0..3][g], i.e. the 16
// consecutive columns 16 g .. 16 g + 15: one 16-byte store per row block and lane.
template <int NW>
__device__ __forceinline__ void store_residues16(const v4i (&acc)[8][4], int64_t m, int64_t n,
                                                 int64_t row0, int64_t col0, int grp, int wq,
                                                 int lane, int mod, double inv,
                                                 int8_t* __restrict__ o, int64_t ldo, bool full,
                                                 int vec_out) {
  auto emit = [&](auto byte_of) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = pack4b(byte_of(acc[i][j][0]), byte_of(acc[i][j][1]), byte_of(acc[i][j][2]),
                      byte_of(acc[i][j][3]));
      const auto r02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
      const auto r13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
      const auto x = __builtin_amdgcn_permlane16_swap(r02[0], r13[0], false, false);
      const auto y = __builtin_amdgcn_permlane16_swap(r02[1], r13[1], false, false);
      const uint4 v = make_uint4(x[0], x[1], y[0], y[1]);
      const int64_t row = row0 + grp * 128 + 16 * i + (lane & 15);
      const int64_t col = col0 + wq * 64 + 16 * (lane >> 4);
      int8_t* dst = o + row * ldo + col;
      if (full) {
        *reinterpret_cast<uint4*>(dst) = v;
      } else if (row < m) {
        if (vec_out && col + 16 <= n) {
          *reinterpret_cast<uint4*>(dst) = v;
        } else {
          const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
          for (int u = 0; u < 16; ++u)
            if (col + u < n) dst[u] = (int8_t)(wv[u >> 2] >> (8 * (u & 3)));
        }
      }
    }
  };
  if (mod == 256) {
    emit([](int v) { return (uint32_t)v; });
  } else {
    const uint32_t um = (uint32_t)mod;
    emit([=](int v) { return residue_byte_odd(v, um, inv); });
  }
}

template <int kEpi, int NW>
__global__ __launch_bounds__(64 * NW, 1) void gemm_i8_pairs_kernel(
    int64_t m, int64_t n, int64_t kp, const int8_t* __restrict__ pa, int64_t stride_a,
    const int8_t* __restrict__ pb, int64_t stride_b, void* __restrict__ out, int64_t ldo,
    int64_t stride_o, int tiles_m, int tiles_n, int tiles, EpiModuli E, int vec_out) {
  __shared__ __attribute__((aligned(1024))) int8_t lds[2 * kPairBytes];

  constexpr int kWaves = NW;
  constexpr int kRegions = kPairBytes / 1024;          // 64 regions of 8 rows x 128 B
  constexpr int kLoadsPerWave = kRegions / NW;         // 8 (NW = 8)
  constexpr int TI = 8, TJ = 4;                        // 16 x 16 blocks of a wave
  constexpr int kStores = kEpi == kEpiProducts ? TI * TJ : TI;  // per full tile
  static_assert(NW == 8 && kStores <= 63, "regions 0..31 are A; the store count fits vmcnt");
  static_assert(kLoadsPerWave == 8, "8 loads in one quarter of 16 MFMAs");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = __builtin_amdgcn_readfirstlane(wave / (NW / 2));   // rows grp * 128
  const int wq = __builtin_amdgcn_readfirstlane(wave % (NW / 2));    // columns wq * 64

  // This workgroup's tiles: first, first + G, ... below tiles (all uniform).
  const int G = gridDim.x;
  const int t_end = tiles;
  const int step = G;
  int t = G % kXcds == 0 ? (int)(blockIdx.x % kXcds) * (G / kXcds) + (int)(blockIdx.x / kXcds)
                         : (int)blockIdx.x;
  if (t >= t_end) return;

  // Tile -> (modulus, tile row, tile column), tile rows grouped by kPairGroupM.
  struct Tile {
    int l;
    int64_t row0, col0;
    uint64_t base_a, base_b;            // tile origins of A_l and B_l (uniform)
    uint32_t voff[kLoadsPerWave];       // per-lane source offsets of the loads
  };
  const int per_mod = tiles_m * tiles_n;
  const int per_group = kPairGroupM * tiles_n;
  // Region rg = wave + NW q: rows 8 (rg % 32) .. +7 of A (q < 4) or B; lane i lands at
  // row 8 (rg % 32) + i / 8, physical chunk i % 8, which holds logical chunk
  // (i % 8) ^ ((row >> 1) & 7); rows past the matrix re-read its last row.
  auto make_tile = [&](int tt, Tile& d) {
    d.l = tt / per_mod;
    const int rem = tt - d.l * per_mod;
    const int first_m = (rem / per_group) * kPairGroupM;
    const int gsize = tiles_m - first_m < kPairGroupM ? tiles_m - first_m : kPairGroupM;
    const int in_group = rem % per_group;
    d.row0 = (int64_t)(first_m + in_group % gsize) * BM;
    d.col0 = (int64_t)(in_group / gsize) * BN;
    d.base_a = (uint64_t)(pa + d.l * stride_a + d.row0 * kp);
    d.base_b = (uint64_t)(pb + d.l * stride_b + d.col0 * kp);
#pragma unroll
    for (int q = 0; q < kLoadsPerWave; ++q) {
      const bool is_b = q >= kLoadsPerWave / 2;
      const int row = 8 * ((wave + kWaves * q) & 31) + (lane >> 3);
      const int chunk = (lane & 7) ^ ((row >> 1) & 7);
      const int64_t origin = is_b ? d.col0 : d.row0;
      const int64_t last = (is_b ? n : m) - 1;
      const int64_t gr = origin + row < last ? origin + row : last;
      d.voff[q] = (uint32_t)((gr - origin) * kp + 16 * chunk);
    }
  };

  const uint32_t lds0 = lds_address(lds);
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(lds0 + wave * 1024);
  const int np = (int)(kp / kPairRow);
  // Load q of pair `pair` of the current tile (next: of the next tile) into LDS buffer
  // `buf`.
  Tile cur, nxt;
  auto load = [&](bool next, int pair, int buf, int q) {
    const uint32_t vo = next ? nxt.voff[q] : cur.voff[q];
    const uint64_t base = q < kLoadsPerWave / 2 ? (next ? nxt.base_a : cur.base_a)
                                                : (next ? nxt.base_b : cur.base_b);
    dma16_sbase(vo, base + (uint64_t)pair * kPairRow,
                wave_lds + (uint32_t)buf * kPairBytes + q * (kWaves * 1024));
  };

  v4i acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0;

  // Fragment rows: A block i at tile row grp * 128 + 16 i + lane % 16, B block j at tile
  // column wq * 64 + 16 j + lane % 16; K half kh holds logical chunks 4 kh .. 4 kh + 3.
  // Blocks start at multiples of 16 rows, so the row swizzle is (lane % 16) / 2 for all.
  const int frow = lane & 15;
  const int fchunk = lane >> 4;
  const int sw = frow >> 1;
  // per K half: this lane's row of A block 0 and of B block 0 plus its swizzled chunk;
  // other blocks are 16 rows (2 KiB) further, a constant offset
  const int oa0 = (grp * 128 + frow) * kPairRow + (((0 + fchunk) ^ sw) << 4);
  const int oa1 = (grp * 128 + frow) * kPairRow + (((4 + fchunk) ^ sw) << 4);
  const int ob0 = BM * kPairRow + (wq * 64 + frow) * kPairRow + (((0 + fchunk) ^ sw) << 4);
  const int ob1 = BM * kPairRow + (wq * 64 + frow) * kPairRow + (((4 + fchunk) ^ sw) << 4);
  v4i fa[2][2][2], fb[2][4];   // fa[set][K half][row block of a quarter], fb[K half][block]
  auto read_a = [&](int set, const int8_t* st, int kh, int rb, int ii) {
    fa[set][kh][ii] = *reinterpret_cast<const v4i*>(st + (kh ? oa1 : oa0) + rb * 16 * kPairRow);
  };
  auto read_b = [&](const int8_t* st, int kh, int idx) {
    fb[kh][idx] = *reinterpret_cast<const v4i*>(st + (kh ? ob1 : ob0) + idx * 16 * kPairRow);
  };
  // Quarter q: MFMA idx is row block 2q + idx / 8, column block (idx / 2) % 4, K half
  // idx % 2, on A set q % 2.  After the first four MFMAs come the reads of the next
  // quarter's A fragments (q < 3: row blocks 2q+2, 2q+3 of stage `st` into the other set;
  // q = 3: row blocks 0, 1 of stage `sn`), in quarter 3 each B fragment is read from `sn`
  // right after its last use, and loads 0 .. nl-1 of pair lp (next tile if `next`) go into
  // buffer lb, one after every second MFMA.
  auto quarter = [&](int q, const int8_t* st, const int8_t* sn, bool next, int lp, int lb,
                     int nl) {
    const int as = q & 1;
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      const int ii = idx >> 3, j = (idx >> 1) & 3, kh = idx & 1;
      acc[2 * q + ii][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fb[kh][j], fa[as][kh][ii],
                                                                 acc[2 * q + ii][j], 0, 0, 0);
      if (idx < 4) {
        if (q < 3) read_a(as ^ 1, st, idx & 1, 2 * (q + 1) + (idx >> 1), idx >> 1);
        else read_a(as ^ 1, sn, idx & 1, idx >> 1, idx >> 1);
      } else if (q == 3 && idx >= 8) {
        read_b(sn, idx & 1, (idx - 8) >> 1);
      }
      if ((idx & 1) == 1 && (idx >> 1) < nl) load(next, lp, lb, idx >> 1);
      __builtin_amdgcn_sched_barrier(0);
      // The wave that reaches the second half of its quarter first is preferred by the
      // SIMD's issue arbiter until the quarter ends, so one of the two waves runs ahead
      // to the next quarter's reads and loads (8192^3, r = 16: 6.837 -> 6.793 ms, mean
      // of five launches each).
      if (idx == 7) __builtin_amdgcn_s_setprio(1);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  make_tile(t, cur);
#pragma unroll
  for (int q = 0; q < kLoadsPerWave; ++q) load(false, 0, 0, q);
#pragma unroll
  for (int q = 0; q < kLoadsPerWave; ++q) load(false, 1, 1, q);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoadsPerWave) : "memory");
  wg_barrier();
#pragma unroll
  for (int idx = 0; idx < 4; ++idx) {
    read_a(0, lds, idx & 1, idx >> 1, idx >> 1);
    read_b(lds, 0, idx);
    read_b(lds, 1, idx);
  }
  int par = 0;                 // LDS buffer of the current tile's pair 0
  bool stores_pending = false; // the previous tile's epilogue issued exactly kStores stores
  for (;;) {
    const int t_next = t + step;
    const bool has_next = t_next < t_end;
    if (has_next) make_tile(t_next, nxt);
    for (int p = 0; p < np; ++p) {
      __builtin_amdgcn_sched_barrier(0);
      const int b0 = (par + p) & 1;      // pair p's buffer (and pair p+2's)
      const int b1 = b0 ^ 1;             // pair p+1's buffer
      const int8_t* st = lds + b0 * kPairBytes;
      const bool last = p + 1 == np;
      quarter(0, st, st, false, 0, 0, 0);
      quarter(1, st, st, false, 0, 0, 0);
      quarter(2, st, st, false, 0, 0, 0);
      // pair p+1 has landed (this wave's loads; the barrier covers the others) and every
      // wave holds its quarter-3 fragments of pair p.  In pair 0 only the previous
      // epilogue's stores may be issued after pair 1's loads.
      if (p == 0 && stores_pending)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kStores) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      wg_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // quarter 3: the first fragments of pair p+1 (the next tile's pair 0 after the last
      // pair; a harmless re-read of pair p after the last tile's), and pair p+2 into pair
      // p's buffer, now free
      const bool wrap = p + 2 >= np;     // pair p+2 belongs to the next tile
      const bool q3_loads = !wrap || has_next;
      const int8_t* sn = last && !has_next ? st : lds + b1 * kPairBytes;
      quarter(3, st, sn, wrap, wrap ? p + 2 - np : p + 2, b0, q3_loads ? kLoadsPerWave : 0);
    }
    // Epilogue of tile `cur`: exactly kStores stores per wave when the tile is full.
    const bool full = vec_out && cur.row0 + BM <= m && cur.col0 + BN <= n;
    if (kEpi == kEpiProducts) {
      // lane l of block (i, j): row 16 i + l % 16, columns 16 j + 4 (l / 16) + 0..3
      int32_t* o = reinterpret_cast<int32_t*>(out) + cur.l * stride_o;
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int64_t row = cur.row0 + grp * 128 + 16 * i + (lane & 15);
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int64_t col = cur.col0 + wq * 64 + 16 * j + 4 * (lane >> 4);
          int32_t* dst = o + row * ldo + col;
          const v4i v = acc[i][j];
          if (full) {
            *reinterpret_cast<v4i*>(dst) = v;
          } else if (row < m) {
            if (vec_out && col + 4 <= n) {
              *reinterpret_cast<v4i*>(dst) = v;
            } else {
              for (int u = 0; u < 4; ++u)
                if (col + u < n) dst[u] = v[u];
            }
          }
        }
      }
    } else {
      store_residues16<NW>(acc, m, n, cur.row0, cur.col0, grp, wq, lane, E.mod[cur.l],
                           E.inv[cur.l], reinterpret_cast<int8_t*>(out) + cur.l * stride_o, ldo,
                           full, vec_out);
    }
    if (!has_next) break;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][v] = 0;
    stores_pending = full;
    par = (par + np) & 1;
    t = t_next;
    cur = nxt;
  }
  // Every load this wave issued has been waited for (the last tile issues none past its
  // last pair); the stores drain on their own.
}

// Compute units of the current device, cached per device.
int compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev >= 0 && dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return -1;
  if (dev >= 0 && dev < 64) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace

int launch_gemm_i8(int64_t m, int64_t n, int64_t kp, int r, const int8_t* pa, int64_t stride_a,
                   const int8_t* pb, int64_t stride_b, void* out, int64_t ldo, int64_t stride_o,
                   int epilogue, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
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
  const int64_t elem = epilogue == kEpiProducts ? 4 : 1;
  const int64_t vbytes = 16;
  const int vec_out = (reinterpret_cast<uintptr_t>(out) % vbytes) == 0 &&
                      (ldo * elem) % vbytes == 0 && (stride_o * elem) % vbytes == 0;
  constexpr int NW = kWavesDefault;
  const dim3 block(64 * NW);
  // whole-line loads need K in steps of 128; the tile pipeline needs two of them
  const bool pairs = kp % kPairRow == 0 && kp >= 2 * kPairRow;
  const int cus = compute_units();
  if (cus <= 0) return OZK_EHIP;
  const dim3 grid((unsigned)blocks);
  const dim3 grid_p((unsigned)(blocks < cus ? blocks : cus));  // one workgroup per CU
  const int tiles = (int)blocks;
#define OZK_GEMM(EPI)                                                                        \
  if (pairs)                                                                                 \
    hipExtLaunchKernelGGL((gemm_i8_pairs_kernel<EPI, NW>), grid_p, block, 0, s, ev_start,    \
                          ev_stop, 0, m, n, kp, pa, stride_a, pb, stride_b, out, ldo,         \
                          stride_o, tiles_m, tiles_n, tiles, E, vec_out);                     \
  else                                                                                       \
    hipExtLaunchKernelGGL((gemm_i8_kernel<EPI, NW>), grid, block, 0, s, ev_start, ev_stop, 0, \
                          m, n, kp, pa, stride_a, pb, stride_b, out, ldo, stride_o, tiles_m,  \
                          tiles_n, E, vec_out)
  if (epilogue == kEpiProducts) {
    OZK_GEMM(kEpiProducts);
  } else {
    OZK_GEMM(kEpiResidues);
  }
#undef OZK_GEMM
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

}  // namespace ozk
