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
// every 16-byte LDS fragment read feeds four MFMAs.  Global tiles are loaded straight
// into a 4-stage LDS ring (128 KiB) by global_load_lds_dwordx4, three K tiles ahead, with
// one barrier per K tile placed between the two MFMA sub-steps (see the pipeline below).
// LDS rows are 64 bytes with the four 16-byte chunks XOR-swizzled by (row >> 2) & 3, so
// the 16 lanes of a fragment read (16 consecutive rows, one chunk each) cover all 64
// banks.  Workgroups are mapped XCD by XCD (the hardware deals them out round-robin over
// the 8 XCDs) onto contiguous runs of tiles, ordered in groups of 4 tile rows, so the
// tiles in flight on one XCD share A rows and B columns in its L2.
//
// Epilogues: the int32 products themselves, or their symmetric residues modulo m_l as
// int8 (what the CRT reconstruction consumes: 1 byte instead of 4 per output), staged
// through LDS so that global stores are 16-byte and coalesced.
#include <type_traits>

#include "lds_dma.h"
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
// (v - q m) mod 2^8, for which the low 24 bits of q suffice (v_mul_u32_u24).
__device__ __forceinline__ uint32_t residue_byte_odd(int v, uint32_t m, double inv) {
  constexpr double kMagicD = 6755399441055744.0;
  const double t = __builtin_fma((double)v, inv, kMagicD);
  const uint32_t q = (uint32_t)__double_as_longlong(t);
  return (uint32_t)v - __umul24(q, m);
}

// Bytes 0 of four words into one word (b0 lowest).
__device__ __forceinline__ uint32_t pack4b(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

constexpr int kStages = 4;
constexpr int kStageBytes = kLdsA + kLdsB;  // 32 KiB: A rows 0..255 then B rows 0..255
constexpr int kRegions = kStageBytes / 1024;  // 1 KiB regions, one per wave instruction
constexpr int kRegionsPerWave = kRegions / 4;

template <int kEpi>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_kernel(
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

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1;   // 0..1: rows wr*128
  const int wc = wave & 1;    // 0..1: cols wc*128

  // Direct-load sources: wave w fills regions w, w+4, ...; region rg holds 16 rows of A
  // (rg < 16) or B, 64 bytes each; lane i lands at row 16*(rg%16) + i/4, physical chunk
  // i%4, which holds logical K chunk (i%4) ^ ((row >> 2) & 3) (the read-side swizzle).
  const int8_t* src[kRegionsPerWave];
#pragma unroll
  for (int q = 0; q < kRegionsPerWave; ++q) {
    const int rg = wave + 4 * q;
    const bool is_b = rg >= 16;
    const int row = 16 * (rg & 15) + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    int64_t gr = (is_b ? col0 : row0) + row;
    const int64_t last = (is_b ? n : m) - 1;
    gr = gr < last ? gr : last;
    src[q] = (is_b ? B : A) + gr * kp + 16 * chunk;
  }
  const uint32_t lds0 = lds_address(lds);
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(lds0 + wave * 1024);
  const int64_t nk = kp / BK;
  auto issue_tile = [&](int64_t t) {  // tile t (clamped to the last) into stage t % kStages
    const int64_t tc = t < nk ? t : nk - 1;
    const uint32_t base = wave_lds + (uint32_t)(t % kStages) * kStageBytes;
#pragma unroll
    for (int q = 0; q < kRegionsPerWave; ++q) dma16(src[q] + tc * BK, base + q * 4096);
  };

  v16i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  // Fragment reads: lane holds row (lane & 31) of a 32-row block and 16 bytes at
  // K offset 32*kk + 16*(lane >> 5); A and B use the same K map, so the product is
  // independent of how the instruction orders K internally.
  const int frow = lane & 31;
  const int fchunk = lane >> 5;
  v4i fa[2][4], fb[2][4];
  auto read_frags = [&](v4i (&xa)[4], v4i (&xb)[4], int64_t t, int kk) {
    const int8_t* la = lds + (t % kStages) * kStageBytes;
    const int8_t* lb = la + kLdsA;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      xa[i] = *reinterpret_cast<const v4i*>(la + swz(wr * 128 + i * 32 + frow, kk * 2 + fchunk));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      xb[j] = *reinterpret_cast<const v4i*>(lb + swz(wc * 128 + j * 32 + frow, kk * 2 + fchunk));
  };

  // One fragment read (idx 0..3: A blocks, 4..7: B blocks) of K half kk of tile t.
  auto frag_read = [&](v4i (&xa)[4], v4i (&xb)[4], int64_t t, int kk, int idx) {
    const int8_t* la = lds + (t % kStages) * kStageBytes;
    if (idx < 4)
      xa[idx] = *reinterpret_cast<const v4i*>(la + swz(wr * 128 + idx * 32 + frow, kk * 2 + fchunk));
    else
      xb[idx - 4] = *reinterpret_cast<const v4i*>(
          la + kLdsA + swz(wc * 128 + (idx - 4) * 32 + frow, kk * 2 + fchunk));
  };

  // Pipeline: tiles t+1 .. t+3 are in flight while tile t is multiplied.
  //   sub-step 0 of tile t: 16 MFMAs on fragments (t, 0), one read of fragments (t, 1)
  //   after every other MFMA;
  //   wait for this wave's loads of tile t+1, barrier (tile t+1 complete from all waves;
  //   every wave is past its reads of tile t-1);
  //   sub-step 1 of tile t: 16 MFMAs on (t, 1), alternately followed by one load of tile
  //   t+3 (into the stage of tile t-1) and one read of fragments (t+1, 0).
  // Every MFMA is followed by at most one memory instruction (pinned by scheduling
  // barriers), so the issue of loads and LDS reads hides behind the matrix pipe.
  issue_tile(0);
  issue_tile(1);
  issue_tile(2);
  asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  read_frags(fa[0], fb[0], 0, 0);
  for (int64_t t = 0; t < nk; ++t) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      const int i = idx >> 2, j = idx & 3;
      acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[0][j], fa[0][i], acc[i][j], 0, 0, 0);
      if ((idx & 1) == 0) frag_read(fa[1], fb[1], t, 1, idx >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int64_t tl = t + 3 < nk ? t + 3 : nk - 1;   // past the end: reload the last tile
    const uint32_t base = wave_lds + (uint32_t)((t + 3) % kStages) * kStageBytes;
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      const int i = idx >> 2, j = idx & 3;
      acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[1][j], fa[1][i], acc[i][j], 0, 0, 0);
      if ((idx & 1) == 0)
        dma16(src[idx >> 1] + tl * BK, base + (idx >> 1) * 4096);
      else
        frag_read(fa[0], fb[0], t + 1, 0, idx >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // The MFMA runs with the B fragment as its first operand, so each accumulator tile is
  // C^T: lane -> row (lane & 31) of the 32 x 32 block of C, register v -> column
  // 8*(v/4) + 4*(lane/32) + (v%4); registers 4q..4q+3 hold 4 consecutive columns.
  const int mod = E.mod[l];
  const double inv = E.inv[l];
  const int64_t wrow0 = row0 + wr * 128, wcol0 = col0 + wc * 128;
  if (kEpi == kEpiProducts) {
    int32_t* o = reinterpret_cast<int32_t*>(out) + l * stride_o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = wrow0 + i * 32 + (lane & 31);
      if (row >= m) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
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
  // Residues: stage the wave's 128 x 128 byte tile in LDS (row pitch 136: the dword writes
  // of 64 lanes and the 8-byte reads of each 16-lane group hit distinct banks), then store
  // rows with 16-byte coalesced writes (8 lanes per 128-byte row segment).
  constexpr int kPitch = 136;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();  // every wave is past its last read of the LDS ring
  int8_t* tile = lds + wave * (128 * kPitch);
  // m = 256 keeps the low byte of the product; odd moduli reduce (uniform branch, taken
  // once per tile rather than per element).
  auto stage = [&](auto byte_of) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w = pack4b(byte_of(acc[i][j][4 * q]), byte_of(acc[i][j][4 * q + 1]),
                                    byte_of(acc[i][j][4 * q + 2]), byte_of(acc[i][j][4 * q + 3]));
          *reinterpret_cast<uint32_t*>(tile + (i * 32 + (lane & 31)) * kPitch + j * 32 + 8 * q +
                                       4 * (lane >> 5)) = w;
        }
  };
  if (mod == 256) {
    stage([](int v) { return (uint32_t)v; });
  } else {
    const uint32_t um = (uint32_t)mod;
    stage([=](int v) { return residue_byte_odd(v, um, inv); });
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave reads back only its own tile
  int8_t* o = reinterpret_cast<int8_t*>(out) + l * stride_o;
#pragma unroll 4
  for (int s8 = 0; s8 < 16; ++s8) {
    const int rl = s8 * 8 + (lane >> 3), cl = 16 * (lane & 7);
    const int64_t row = wrow0 + rl, col = wcol0 + cl;
    const int8_t* srcp = tile + rl * kPitch + cl;
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
  const int64_t elem = epilogue == kEpiProducts ? 4 : 1;
  const int64_t vbytes = 16;
  const int vec_out = (reinterpret_cast<uintptr_t>(out) % vbytes) == 0 &&
                      (ldo * elem) % vbytes == 0 && (stride_o * elem) % vbytes == 0;
  if (epilogue == kEpiProducts)
    hipLaunchKernelGGL(gemm_i8_kernel<kEpiProducts>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       s, m, n, kp, pa, stride_a, pb, stride_b, out, ldo, stride_o, tiles_m,
                       tiles_n, E, vec_out);
  else
    hipLaunchKernelGGL(gemm_i8_kernel<kEpiResidues>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       s, m, n, kp, pa, stride_a, pb, stride_b, out, ldo, stride_o, tiles_m,
                       tiles_n, E, vec_out);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

}  // namespace ozk
