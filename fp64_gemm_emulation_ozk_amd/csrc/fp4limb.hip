// Exact INT8 x INT8 matrix products through base-13 FP4 limbs on the gfx950 scaled
// f8f6f4 MFMA.  [AWE] (arXiv 2609.24519 listing, English abstract): the FP4 values
// doubled form S = {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12}, which holds every residue
// mod 13, so an integer splits with carries into base-13 digits in S; an INT8 operand
// takes 3 digits with weights (1, 13, 169) and the product is the sum of the 9 pairwise
// digit products weighted by 13^(da+db).
//
// Digits: the digit of residue rho is the element of S of least magnitude congruent to
// rho mod 13 (so |d0|, |d1| <= 8 and d2 in {-1, 0, 1}); a digit d is stored as the e2m1
// code of d/2, two codes per byte with the even K index in the low nibble.
//
// Products: v_mfma_scale_f32 f8f6f4 MFMAs with both operands in e2m1 and both E8M0
// block scales equal to 2^1, so every elementary product is the integer d_a d_b.  The 9
// digit products are summed per weight class w = da + db (5 fp32 accumulators).  Each
// K element adds at most 128 in magnitude to any class (class 1: |d0 d1| + |d1 d0|), so
// for K <= 131071 every partial sum is an integer below 2^24 and fp32 holds it exactly;
// the classes are then converted to integers and combined with weights 1, 13, 169, 2197,
// 28561 in wrap-around 32-bit arithmetic (the exact result fits int32: |C| <= 2^14 K).
#include <type_traits>

#include "fp4_pack.h"
#include "lds_dma.h"
#include "ozk_internal.h"

namespace ozk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ digit table
constexpr int e2m1_twice(int code) {  // 2 * value of an e2m1 code (an integer in S)
  const int e = (code >> 1) & 3, mbit = code & 1;
  const int mag2 = e == 0 ? mbit : (1 << e) + (mbit << (e - 1));  // 2 * 2^(e-1) (1 + m/2)
  return (code & 8) ? -mag2 : mag2;
}

constexpr int code_of_digit(int d) {
  for (int c = 0; c < 16; ++c)
    if (e2m1_twice(c) == d) return c;  // the first hit for 0 is code 0 (+0)
  return -1;
}

constexpr int digit_of_residue(int rho) {
  int best = 100;
  for (int c = 0; c < 16; ++c) {
    const int d = e2m1_twice(c);
    if (((d % 13) + 13) % 13 == rho && (d < 0 ? -d : d) < (best < 0 ? -best : best)) best = d;
  }
  return best;
}

struct LimbTable {
  uint16_t codes[256];  // index x + 128: code(d0) | code(d1) << 4 | code(d2) << 8
};

constexpr LimbTable make_limb_table() {
  LimbTable t{};
  for (int x = -128; x < 128; ++x) {
    const int d0 = digit_of_residue(((x % 13) + 13) % 13);
    const int x1 = (x - d0) / 13;
    const int d1 = digit_of_residue(((x1 % 13) + 13) % 13);
    const int d2 = (x1 - d1) / 13;
    t.codes[x + 128] = (uint16_t)(code_of_digit(d0) | (code_of_digit(d1) << 4) |
                                  (code_of_digit(d2) << 8));
  }
  return t;
}

__constant__ LimbTable d_limbs = make_limb_table();
static_assert(make_limb_table().codes[128] == 0, "0 splits into three zero digits");

// ------------------------------------------------------------------ packer
// A packer's table in LDS: the spread word (byte d = code of digit plane d) of every
// value, indexed by the unsigned byte of the stored value.
__device__ __forceinline__ void load_limb_lut(uint32_t* lut) {
  if (threadIdx.x < 256) lut[threadIdx.x] = spread_nibbles(d_limbs.codes[threadIdx.x ^ 0x80]);
  __syncthreads();
}

// 32 consecutive K values -> 16 bytes per digit plane; at(h) is the unsigned byte of
// value h.
template <typename At>
__device__ __forceinline__ void pack32(At at, const uint32_t* lut, uint4 (&out)[3]) {
  uint32_t w[3][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t sw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) sw[u] = lut[at(8 * q + u)];
    uint32_t o[3];
    pack8_planes<3>(sw, o);
#pragma unroll
    for (int d = 0; d < 3; ++d) w[d][q] = o[d];
  }
#pragma unroll
  for (int d = 0; d < 3; ++d) out[d] = make_uint4(w[d][0], w[d][1], w[d][2], w[d][3]);
}

// axis 0: x rows x cols (K = cols); thread -> (row, 32-value chunk).
// vec: x and ldx are 16-byte aligned, so a whole 32-value chunk is two 16-byte loads.
__global__ __launch_bounds__(256) void pack_rows_kernel(const int8_t* __restrict__ x,
                                                        int64_t rows, int64_t cols, int64_t ldx,
                                                        uint8_t* __restrict__ planes,
                                                        int64_t ldpb, int64_t plane_stride,
                                                        int vec) {
  __shared__ uint32_t lut[256];
  load_limb_lut(lut);
  const int64_t chunks = ldpb / 16;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= rows * chunks) return;
  const int64_t row = g / chunks;
  const int64_t h0 = (g - row * chunks) * 32;
  const int8_t* src = x + row * ldx;
  uint32_t d[8];   // byte h & 3 of d[h >> 2] = value h0 + h
  if (vec && h0 + 32 <= cols) {
    const uint4 w0 = *reinterpret_cast<const uint4*>(src + h0);
    const uint4 w1 = *reinterpret_cast<const uint4*>(src + h0 + 16);
    d[0] = w0.x; d[1] = w0.y; d[2] = w0.z; d[3] = w0.w;
    d[4] = w1.x; d[5] = w1.y; d[6] = w1.z; d[7] = w1.w;
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t w = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (h0 + 4 * q + c < cols) w |= (uint32_t)(uint8_t)src[h0 + 4 * q + c] << (8 * c);
      d[q] = w;
    }
  }
  uint4 out[3];
  pack32([&](int h) { return byte_of(d[h >> 2], h & 3, 255u); }, lut, out);
#pragma unroll
  for (int dd = 0; dd < 3; ++dd)
    *reinterpret_cast<uint4*>(planes + dd * plane_stride + row * ldpb + h0 / 2) = out[dd];
}

// axis 1: x rows x cols with K = rows; thread -> (4 consecutive columns, 32-value chunk of
// K).  The 64 threads of a wave take 256 consecutive columns, so with vec (x and ldx 4-byte
// aligned) every load instruction reads 256 consecutive bytes of one row; the 8 waves of a
// block take 8 consecutive chunks, so each 128-byte line of a plane is written whole by one
// block (with 4 waves per block two blocks shared every line: 1.33x the algorithmic bytes).
__global__ __launch_bounds__(512) void pack_cols_kernel(const int8_t* __restrict__ x,
                                                        int64_t rows, int64_t cols, int64_t ldx,
                                                        uint8_t* __restrict__ planes,
                                                        int64_t ldpb, int64_t plane_stride,
                                                        int vec) {
  __shared__ uint32_t lut[256];
  load_limb_lut(lut);
  const int64_t col0 = 4 * ((int64_t)blockIdx.x * 64 + (threadIdx.x & 63));
  const int64_t h0 = ((int64_t)blockIdx.y * 8 + (threadIdx.x >> 6)) * 32;
  if (col0 >= cols || h0 >= 2 * ldpb) return;
  const bool full = vec && col0 + 4 <= cols;
  uint32_t r[32];   // byte c of r[h] = row h0 + h, column col0 + c (0 past the matrix)
#pragma unroll
  for (int h = 0; h < 32; ++h) {
    uint32_t w = 0;
    if (h0 + h < rows) {
      const int8_t* p = x + (h0 + h) * ldx + col0;
      if (full) {
        w = *reinterpret_cast<const uint32_t*>(p);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (col0 + c < cols) w |= (uint32_t)(uint8_t)p[c] << (8 * c);
      }
    }
    r[h] = w;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (col0 + c >= cols) break;
    uint4 out[3];
    pack32([&](int h) { return byte_of(r[h], c, 255u); }, lut, out);
#pragma unroll
    for (int dd = 0; dd < 3; ++dd)
      *reinterpret_cast<uint4*>(planes + dd * plane_stride + (col0 + c) * ldpb + h0 / 2) =
          out[dd];
  }
}

__device__ __forceinline__ v16f mfma_fp4(const v4i& a, const v4i& b, const v16f& c) {
  const v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  // cbsz = blgp = 4: both operands e2m1; scales 0x80 = 2^1 (E8M0) on both sides.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, 0x80, 0, 0x80);
}

typedef float v4f __attribute__((ext_vector_type(4)));

// The same on v_mfma_scale_f32_16x16x128_f8f6f4: lane (row lane % 16, chunk lane / 16)
// holds 32 codes of its row, A and B alike; lane l of the result holds column l % 16,
// rows 4 (l / 16) + 0..3.
__device__ __forceinline__ v4f mfma_fp4_16(const v4i& a, const v4i& b, const v4f& c) {
  const v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 4, 0, 0x80, 0, 0x80);
}

// ------------------------------------------------------------------ 9 products (test path)
// One wave per 32 x 32 output block; fragments straight from global memory.  Lane
// (row = lane & 31, half = lane >> 5) supplies the 16 bytes (32 codes) at byte offset
// 32*step + 16*half of its row, identically for A and B.
__global__ __launch_bounds__(64) void limb_products_kernel(
    int64_t m, int64_t n, int64_t ldpb, const uint8_t* __restrict__ pa, int64_t stride_a,
    const uint8_t* __restrict__ pb, int64_t stride_b, int32_t* __restrict__ out, int64_t ldo,
    int64_t stride_o) {
  const int lane = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.y * 32, col0 = (int64_t)blockIdx.x * 32;
  int64_t ra = row0 + (lane & 31), rb = col0 + (lane & 31);
  ra = ra < m ? ra : m - 1;
  rb = rb < n ? rb : n - 1;
  const int half = lane >> 5;
  v16f acc[9];
#pragma unroll
  for (int q = 0; q < 9; ++q)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[q][v] = 0.0f;
  for (int64_t k0 = 0; k0 < ldpb; k0 += 32) {
    v4i fa[3], fb[3];
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      fa[d] = *reinterpret_cast<const v4i*>(pa + d * stride_a + ra * ldpb + k0 + 16 * half);
      fb[d] = *reinterpret_cast<const v4i*>(pb + d * stride_b + rb * ldpb + k0 + 16 * half);
    }
#pragma unroll
    for (int da = 0; da < 3; ++da)
#pragma unroll
      for (int db = 0; db < 3; ++db) acc[3 * da + db] = mfma_fp4(fa[da], fb[db], acc[3 * da + db]);
  }
  const int64_t col = col0 + (lane & 31);
  if (col >= n) return;
#pragma unroll
  for (int q = 0; q < 9; ++q)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = row0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (row < m) out[q * stride_o + row * ldo + col] = (int32_t)acc[q][v];
    }
}

// ------------------------------------------------------------------ fused weighted GEMM
// Workgroup tile 128 x 128, K step 128 codes (64 bytes per row per digit plane), 512
// threads = 8 waves in 2 x 4, each wave 64 x 32 outputs = 4 x 2 blocks of 16 x 16 on
// v_mfma_scale_f32_16x16x128_f8f6f4 (one MFMA takes the whole K step; on random codes
// this shape sustains about 10 % more operations under the board's power limit than
// 32 x 32 x 64), each block with 5 weight-class accumulators (160 registers).  The three
// digit planes of A and of B (48 KiB per K step) are loaded straight into a 3-stage LDS
// ring by global_load_lds_dwordx4, two K steps ahead; every load instruction covers 16
// rows x 64 bytes (16 lines, where 32-byte row pieces would touch 32 lines for the same
// kilobyte).  LDS rows are 64 bytes with the four 16-byte chunks XOR-swizzled by
// (row >> 1) & 3, so the 16 lanes of a fragment read (16 rows, one chunk) cover all 64
// banks (a swizzle by (row >> 2) & 3, also a bijection over 16 rows, measured 152 M bank
// conflict cycles per 8192^3 product; this one none).  A K step runs as four quarters of 18 MFMAs, one per row block (both column
// blocks, the 9 digit pairs, the column blocks alternating so that the MFMAs chaining on
// one class accumulator stand four apart); quarters 0..2 read the next row block's A
// fragments between their MFMAs.  After quarter 2 the wave waits for its loads (those of
// step t+1) and its reads, and one barrier makes step t+1 complete and step t fully read;
// quarter 3 then issues the 6 loads of step t+2 into the stage of step t-1 (past the last
// step the last step is loaded again) and reads step t+1's first A row block and both B
// blocks.  Workgroups are dealt out XCD by XCD onto contiguous runs of tiles grouped by 4
// tile rows, so the tiles in flight on one XCD share A rows and B columns in its L2.
constexpr int FBM = 128, FBN = 128, FROW = 64;  // bytes per row per plane per K step
constexpr int kFThreads = 512;
constexpr int kFPlane = 128 * FROW;              // 8 KiB: one digit plane of A or B
constexpr int kStage = 6 * kFPlane;              // 48 KiB: A planes 0..2, then B planes
constexpr int kFStages = 3;
constexpr int kFGroupM = 4;
constexpr int kFXcds = 8;

// 16 lanes read rows r..r+15 at one logical chunk; rows with equal (row mod 4) share
// banks without the XOR (gfx950 LDS: 64 four-byte banks, 16 lanes of 16 bytes per clock).
__device__ __forceinline__ int fsw_of(int row) { return (row >> 1) & 3; }
__device__ __forceinline__ int fswz(int row, int chunk) {
  return row * FROW + ((chunk ^ fsw_of(row)) << 4);
}

__global__ __launch_bounds__(kFThreads, 1) void fp4_gemm_kernel(
    int64_t m, int64_t n, int64_t ldpb, const uint8_t* __restrict__ pa, int64_t stride_a,
    const uint8_t* __restrict__ pb, int64_t stride_b, int32_t* __restrict__ c, int64_t ldc,
    int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kFStages * kStage];

  // Block -> tile: XCD-contiguous, then grouped by kFGroupM tile rows.
  const int total = gridDim.x;
  int bid = blockIdx.x;
  if (total % kFXcds == 0) bid = (bid % kFXcds) * (total / kFXcds) + bid / kFXcds;
  const int per_group = kFGroupM * tiles_n;
  const int first_m = (bid / per_group) * kFGroupM;
  const int gsize = tiles_m - first_m < kFGroupM ? tiles_m - first_m : kFGroupM;
  const int in_group = bid % per_group;
  const int tm = first_m + in_group % gsize;
  const int tn = in_group / gsize;
  const int64_t row0 = (int64_t)tm * FBM, col0 = (int64_t)tn * FBN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 2;  // 0..1: rows wr*64
  const int wc = wave & 3;   // 0..3: cols wc*32

  // Direct loads: load q (0..5) of a wave fills rows 16*wave .. +15 of plane q (q < 3: A
  // digit q, else B digit q - 3); lane i lands at row 16*wave + i/4, physical chunk i%4,
  // which holds logical chunk (i%4) ^ fsw_of(row).  Rows past the matrix edge read its
  // last row.
  const int lrow = 16 * wave + (lane >> 2);
  const int lchunk = (lane & 3) ^ fsw_of(lrow);
  const int64_t ra = row0 + lrow < m - 1 ? row0 + lrow : m - 1;
  const int64_t rb = col0 + lrow < n - 1 ? col0 + lrow : n - 1;
  const uint32_t voff_a = (uint32_t)((ra - row0) * ldpb + 16 * lchunk);
  const uint32_t voff_b = (uint32_t)((rb - col0) * ldpb + 16 * lchunk);
  const uint64_t base_a = (uint64_t)(pa + row0 * ldpb), base_b = (uint64_t)(pb + col0 * ldpb);
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(lds_address(lds) + wave * 1024);
  const int nk = (int)(ldpb / FROW);
  // Load q of K step tk into the stage of step ts (ts = tk except past the last step, where
  // the last step is loaded again into the stage that step ts would use).
  auto issue_one = [&](int q, int tk, int ts) {
    const uint64_t kb = (uint64_t)tk * FROW;
    const uint32_t dst = wave_lds + (uint32_t)(ts % kFStages) * kStage + q * kFPlane;
    if (q < 3)
      dma16_sbase(voff_a, base_a + (uint64_t)(q * stride_a) + kb, dst);
    else
      dma16_sbase(voff_b, base_b + (uint64_t)((q - 3) * stride_b) + kb, dst);
  };

  v4f acc[4][2][5];   // [row block][column block][weight class]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int w = 0; w < 5; ++w)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][w][v] = 0.0f;

  // Fragments of a 16-row block: lane (row lane & 15, chunk lane >> 4) = 32 codes of the
  // step's 128, the same map for A and B.
  const int frow = lane & 15, fch = lane >> 4;
  auto read_a = [&](v4i& x, int t, int rbk, int d) {
    x = *reinterpret_cast<const v4i*>(lds + (t % kFStages) * kStage + d * kFPlane +
                                      fswz(wr * 64 + rbk * 16 + frow, fch));
  };
  auto read_b = [&](v4i& x, int t, int cbk, int d) {
    x = *reinterpret_cast<const v4i*>(lds + (t % kFStages) * kStage + (3 + d) * kFPlane +
                                      fswz(wc * 32 + cbk * 16 + frow, fch));
  };

  v4i fa[2][3], fb[2][2][3];   // fa[set][digit]; fb[set][col block][digit]
#pragma unroll
  for (int q = 0; q < 6; ++q) issue_one(q, 0, 0);
  if (nk > 1) {
#pragma unroll
    for (int q = 0; q < 6; ++q) issue_one(q, 1, 1);
    asm volatile("s_waitcnt vmcnt(6)" ::: "memory");  // step 0 complete
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    read_a(fa[0][d], 0, 0, d);
    read_b(fb[0][0][d], 0, 0, d);
    read_b(fb[0][1][d], 0, 1, d);
  }
  // 18 MFMAs of row block i (A set as, B set bs); after MFMA idx, optional reads and loads.
  auto quarter = [&](int i, int as, int bs, auto&& after) {
    // Per column block the 9 digit pairs in the order of their weight class, so that the
    // products of one class accumulate back to back (8192^3: 1.851 -> 1.838 ms per call
    // against alternating column blocks, bit-identical).
    constexpr int kDa[9] = {0, 0, 1, 0, 1, 2, 1, 2, 2};
    constexpr int kDb[9] = {0, 1, 0, 2, 1, 0, 2, 1, 2};
#pragma unroll
    for (int idx = 0; idx < 18; ++idx) {
      const int j = idx / 9, da = kDa[idx % 9], db = kDb[idx % 9];
      acc[i][j][da + db] = mfma_fp4_16(fa[as][da], fb[bs][j][db], acc[i][j][da + db]);
      after(idx);
      __builtin_amdgcn_sched_barrier(0);
      // The wave that reaches the second half of a quarter first is preferred by the
      // SIMD's issue arbiter until the quarter ends (8192^3: 1.757 -> 1.743 ms per call,
      // medians of 14 rounds on one board).
      if (idx == 8) __builtin_amdgcn_s_setprio(1);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // One K step; `s` (the B set of step t, t & 1) is a compile-time constant.  Quarters
  // 0..2 (row blocks 0..2) read the next row block's A fragments into the other A set.
  auto kstep = [&](int t, auto s_tag) {
    constexpr int s = decltype(s_tag)::value;
    __builtin_amdgcn_sched_barrier(0);
    quarter(0, 0, s, [&](int idx) { if (idx % 6 == 0) read_a(fa[1][idx / 6], t, 1, idx / 6); });
    quarter(1, 1, s, [&](int idx) { if (idx % 6 == 0) read_a(fa[0][idx / 6], t, 2, idx / 6); });
    quarter(2, 0, s, [&](int idx) { if (idx % 6 == 0) read_a(fa[1][idx / 6], t, 3, idx / 6); });
    // Every load of this wave (those of step t+1) and every read complete; after the
    // barrier step t+1 is complete in LDS and every wave is done with step t's stage.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int tl = t + 2 < nk ? t + 2 : nk - 1;
    const int tn1 = t + 1 < nk ? t + 1 : t;  // past the last step: harmless re-read
    // Quarter 3 (row block 3): the 6 loads of step t+2 after the even MFMAs, and step
    // t+1's A row block 0 and both B blocks after the odd ones.
    quarter(3, 1, s, [&](int idx) {
      if (idx % 2 == 0 && idx < 12) issue_one(idx / 2, tl, t + 2);
      if (idx % 2 == 1) {
        const int r = idx / 2;
        if (r < 3) read_a(fa[0][r], tn1, 0, r);
        else if (r < 6) read_b(fb[s ^ 1][0][r - 3], tn1, 0, r - 3);
        else read_b(fb[s ^ 1][1][r - 6], tn1, 1, r - 6);
      }
    });
  };
  for (int t = 0; t < nk; t += 2) {
    kstep(t, std::integral_constant<int, 0>{});
    if (t + 1 < nk) kstep(t + 1, std::integral_constant<int, 1>{});
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // lane l of block (i, j): column 16 j + l % 16, rows 16 i + 4 (l / 16) + 0..3; the
  // classes are exact integers, combined in wrap-around 32-bit arithmetic.
  constexpr uint32_t kW[5] = {1u, 13u, 169u, 2197u, 28561u};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t col = col0 + wc * 32 + j * 16 + (lane & 15);
    if (col >= n) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = row0 + wr * 64 + i * 16 + 4 * (lane >> 4) + v;
        if (row >= m) continue;
        uint32_t sum = 0;
#pragma unroll
        for (int w = 0; w < 5; ++w) sum += kW[w] * (uint32_t)(int32_t)acc[i][j][w][v];
        c[row * ldc + col] = (int32_t)sum;
      }
  }
}

}  // namespace

int launch_fp4_pack(const int8_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                    uint8_t* planes, int64_t ldpb, int64_t plane_stride, hipStream_t s) {
  if (axis == 0) {
    if (rows <= 0) return OZK_OK;
    const int64_t threads = rows * (ldpb / 16);
    const int vec = (reinterpret_cast<uintptr_t>(x) % 16) == 0 && ldx % 16 == 0;
    hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       x, rows, cols, ldx, planes, ldpb, plane_stride, vec);
  } else {
    if (cols <= 0) return OZK_OK;
    const int vec = (reinterpret_cast<uintptr_t>(x) % 4) == 0 && ldx % 4 == 0;
    dim3 grid((unsigned)((cols + 255) / 256), (unsigned)((2 * ldpb / 32 + 7) / 8));
    hipLaunchKernelGGL(pack_cols_kernel, grid, dim3(512), 0, s, x, rows, cols, ldx, planes, ldpb,
                       plane_stride, vec);
  }
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

int launch_fp4_products(int64_t m, int64_t n, int64_t ldpb, const uint8_t* pa, int64_t stride_a,
                        const uint8_t* pb, int64_t stride_b, int32_t* out, int64_t ldo,
                        int64_t stride_o, hipStream_t s) {
  if (m <= 0 || n <= 0) return OZK_OK;
  dim3 grid((unsigned)((n + 31) / 32), (unsigned)((m + 31) / 32));
  hipLaunchKernelGGL(limb_products_kernel, grid, dim3(64), 0, s, m, n, ldpb, pa, stride_a, pb,
                     stride_b, out, ldo, stride_o);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

int launch_fp4_gemm(int64_t m, int64_t n, int64_t ldpb, const uint8_t* pa, int64_t stride_a,
                    const uint8_t* pb, int64_t stride_b, int32_t* c, int64_t ldc, hipStream_t s) {
  if (m <= 0 || n <= 0) return OZK_OK;
  // K steps of 64 bytes per row; 32-bit lane offsets within a 128-row tile.
  if (ldpb % FROW != 0 || ldpb <= 0 || 128 * ldpb >= (int64_t)1 << 31) return OZK_EINVAL;
  const int64_t tiles_m = (m + FBM - 1) / FBM, tiles_n = (n + FBN - 1) / FBN;
  if (tiles_m * tiles_n > 0x7fffffff) return OZK_EUNSUPPORTED;
  hipLaunchKernelGGL(fp4_gemm_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kFThreads), 0, s,
                     m, n, ldpb, pa, stride_a, pb, stride_b, c, ldc, (int)tiles_m, (int)tiles_n);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

}  // namespace ozk
