// Exact INT8 x INT8 matrix products in 6 FP4 products on the gfx950 scaled f8f6f4 MFMA.
// [AWE] (arXiv 2609.24519 listing, English abstract): with free integer limb weights and
// stored planes that are linear combinations of limbs, an INT8 x INT8 product takes 6 FP4
// matrix products instead of the 9 of base-13 limbs.
//
// Encoding: x = a0 + 29 a1 + 37 a2 with every limb a_i in S = 2 x FP4 = {0, +-1, +-2, +-3,
// +-4, +-6, +-8, +-12} and every pairwise sum a_i + a_j in S as well; among the triples
// that encode x the one taken minimises the largest magnitude of its six plane values
// (a0, a1, a2, a0+a1, a0+a2, a1+a2), then their sum of squares, then (a0, a1, a2)
// lexicographically.  For these weights every plane value is at most 6 in magnitude.
// With u(x), v(y) the six plane values of x and y, the three-term Karatsuba identity gives
//     x y = sum_t coef_t u_t(x) v_t(y),  coef = (c0, c1, c2, w0 w1, w0 w2, w1 w2),
//     c_i = w_i^2 - w_i sum_{j != i} w_j = (-65, -261, 259),
// so C = A B = sum_t coef_t U_t(A) V_t(B): six plane products.  Each plane product is an
// e2m1 x e2m1 MFMA with both E8M0 block scales 2^1 (plane value d stored as the code of
// d/2), so every elementary product is the integer u v, |u v| <= 36, and fp32 sums are
// exact for K <= 466033; the weighted sum is taken in wrap-around 32-bit integers (the
// exact result fits int32).
//
// Layout of the packed planes (per line: a row of A, a column of B): K in steps of 64
// codes; step s of line i occupies bytes 192 s .. 192 s + 191 of the line, plane t at
// byte 32 t of the step, two codes per byte with the even K index in the low nibble.  A
// K step of a whole 128-line tile is then 128 contiguous 192-byte pieces.
#include "fp4_pack.h"
#include "lds_dma.h"
#include "ozk_internal.h"

namespace ozk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kW1 = 29, kW2 = 37;
constexpr int kPlanes = 6;
constexpr int kStepCodes = 64;
constexpr int kStepBytes = kPlanes * kStepCodes / 2;   // 192
constexpr int kCoef[kPlanes] = {1 - kW1 - kW2, kW1 * kW1 - kW1 * (1 + kW2),
                                kW2 * kW2 - kW2 * (1 + kW1), kW1, kW2, kW1 * kW2};
static_assert(kCoef[0] == -65 && kCoef[1] == -261 && kCoef[2] == 259 && kCoef[5] == 1073,
              "Karatsuba coefficients of the weights (1, 29, 37)");

// ------------------------------------------------------------------ encoding table
constexpr int twice_e2m1(int code) {  // 2 x the value of an e2m1 code: an integer in S
  const int e = (code >> 1) & 3, mbit = code & 1;
  const int mag = e == 0 ? mbit : (1 << e) + (mbit << (e - 1));
  return (code & 8) ? -mag : mag;
}

// code_of.c[d + 24]: the e2m1 code of d/2 for d in [-24, 24] (+0 for 0), -1 where d is not
// in S.
struct CodeOf {
  int c[49];
};
constexpr CodeOf make_code_of() {
  CodeOf t{};
  for (int d = 0; d < 49; ++d) t.c[d] = -1;
  for (int code = 15; code >= 0; --code) t.c[twice_e2m1(code) + 24] = code;  // code 0 last
  return t;
}
constexpr CodeOf kCodeOf = make_code_of();

constexpr int code_for(int d) { return d < -24 || d > 24 ? -1 : kCodeOf.c[d + 24]; }

constexpr int iabs(int v) { return v < 0 ? -v : v; }

struct AweTable {
  uint32_t codes[256];  // index x + 128: code of plane t in bits 4t .. 4t + 3
};

constexpr AweTable make_awe_table() {
  AweTable t{};
  for (int x = -128; x < 128; ++x) {
    int best[3] = {0, 0, 0};
    int best_key[5] = {1 << 20, 0, 0, 0, 0};
    for (int c1 = 0; c1 < 16; ++c1) {
      if (c1 == 8) continue;  // -0: the same value as code 0
      for (int c2 = 0; c2 < 16; ++c2) {
        if (c2 == 8) continue;
        const int a1 = twice_e2m1(c1), a2 = twice_e2m1(c2);
        const int a0 = x - kW1 * a1 - kW2 * a2;
        if (code_for(a0) < 0) continue;
        const int v[kPlanes] = {a0, a1, a2, a0 + a1, a0 + a2, a1 + a2};
        bool ok = true;
        int mx = 0, sq = 0;
        for (int q = 0; q < kPlanes; ++q) {
          if (code_for(v[q]) < 0) ok = false;
          mx = iabs(v[q]) > mx ? iabs(v[q]) : mx;
          sq += v[q] * v[q];
        }
        if (!ok) continue;
        const int key[5] = {mx, sq, a0, a1, a2};
        bool less = false;
        for (int q = 0; q < 5; ++q) {
          if (key[q] != best_key[q]) {
            less = key[q] < best_key[q];
            break;
          }
        }
        if (less) {
          for (int q = 0; q < 5; ++q) best_key[q] = key[q];
          best[0] = a0;
          best[1] = a1;
          best[2] = a2;
        }
      }
    }
    const int v[kPlanes] = {best[0], best[1], best[2], best[0] + best[1], best[0] + best[2],
                            best[1] + best[2]};
    uint32_t w = 0;
    for (int q = 0; q < kPlanes; ++q) w |= (uint32_t)code_for(v[q]) << (4 * q);
    t.codes[x + 128] = w;
  }
  return t;
}

__constant__ AweTable d_awe = make_awe_table();
static_assert(make_awe_table().codes[128] == 0, "0 encodes as six zero planes");

// ------------------------------------------------------------------ packers
// A packer's table in LDS, indexed by the unsigned byte of the stored value: the spread
// words (byte t = code of plane t) of planes 0..3 and of planes 4..5.
__device__ __forceinline__ void load_awe_lut(uint2* lut) {
  const uint32_t c = d_awe.codes[threadIdx.x ^ 0x80];   // 256 threads
  lut[threadIdx.x] = make_uint2(spread_nibbles(c & 0xFFFFu), spread_nibbles(c >> 16));
  __syncthreads();
}

// 64 consecutive K values of one line -> the 192 bytes of its K step as 12 pieces of 16
// (piece 2 t + half: plane t, values 32 half .. 32 half + 31); at(h) is the unsigned byte
// of value h.
template <typename At>
__device__ __forceinline__ void pack_step(At at, const uint2* lut, uint4 (&piece)[12]) {
  uint32_t w[kPlanes][8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint2 e = lut[at(8 * q + u)];
      lo[u] = e.x;
      hi[u] = e.y;
    }
    uint32_t o[4], o2[2];
    pack8_planes<4>(lo, o);
    pack8_planes<2>(hi, o2);
#pragma unroll
    for (int t = 0; t < 4; ++t) w[t][q] = o[t];
    w[4][q] = o2[0];
    w[5][q] = o2[1];
  }
#pragma unroll
  for (int t = 0; t < kPlanes; ++t) {
    piece[2 * t] = make_uint4(w[t][0], w[t][1], w[t][2], w[t][3]);
    piece[2 * t + 1] = make_uint4(w[t][4], w[t][5], w[t][6], w[t][7]);
  }
}

// Per-block LDS of the packers: the table and, per wave, 64 staged K steps and their
// destinations.
struct AwePackShared {
  uint2 lut[256];
  uint4 stage[4][64 * 12];
  uint8_t* dsts[4][64];
};

// axis 0: x rows x cols (K = cols); thread -> (row, K step); consecutive threads take
// consecutive steps of a row, so the staged stores of a wave write 12 KiB runs.  vec: x
// and ldx 16-byte aligned, so a whole step of 64 values is four 16-byte loads.
__global__ __launch_bounds__(256) void awe_pack_rows_kernel(const int8_t* __restrict__ x,
                                                            int64_t rows, int64_t cols,
                                                            int64_t ldx, uint8_t* __restrict__ out,
                                                            int64_t ld_line, int64_t steps,
                                                            int vec) {
  __shared__ AwePackShared sh;
  load_awe_lut(sh.lut);
  const int wave = threadIdx.x >> 6;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t wave_g0 = g - (threadIdx.x & 63);
  if (wave_g0 >= rows * steps) return;            // the whole wave is past the end
  const bool valid = g < rows * steps;
  const int64_t gg = valid ? g : wave_g0;           // lanes past the end pack a copy
  const int64_t row = gg / steps;
  const int64_t s = gg - row * steps;
  const int64_t h0 = s * kStepCodes;
  const int8_t* src = x + row * ldx;
  uint32_t d[16];   // byte h & 3 of d[h >> 2] = value h0 + h
  if (vec && h0 + 64 <= cols) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 w = *reinterpret_cast<const uint4*>(src + h0 + 16 * q);
      d[4 * q] = w.x;
      d[4 * q + 1] = w.y;
      d[4 * q + 2] = w.z;
      d[4 * q + 3] = w.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      uint32_t w = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (h0 + 4 * q + c < cols) w |= (uint32_t)(uint8_t)src[h0 + 4 * q + c] << (8 * c);
      d[q] = w;
    }
  }
  uint4 piece[12];
  pack_step([&](int h) { return byte_of(d[h >> 2], h & 3, 255u); }, sh.lut, piece);
  wave_staged_store<12>(sh.stage[wave], sh.dsts[wave], piece,
                        valid ? out + row * ld_line + s * kStepBytes : nullptr);
}

// axis 1: x rows x cols with K = rows; thread -> (4 consecutive columns, K step).  The 64
// threads of a wave take 256 consecutive columns, so with vec (x and ldx 4-byte aligned)
// every load instruction reads 256 consecutive bytes of one row; each of the 4 column
// rounds stores whole 192-byte steps through the staging area.
__global__ __launch_bounds__(256) void awe_pack_cols_kernel(const int8_t* __restrict__ x,
                                                            int64_t rows, int64_t cols,
                                                            int64_t ldx, uint8_t* __restrict__ out,
                                                            int64_t ld_line, int64_t steps,
                                                            int vec) {
  __shared__ AwePackShared sh;
  load_awe_lut(sh.lut);
  const int wave = threadIdx.x >> 6;
  const int64_t col0 = 4 * ((int64_t)blockIdx.x * 64 + (threadIdx.x & 63));
  const int64_t s = (int64_t)blockIdx.y * 4 + wave;
  if (s >= steps || 4 * (int64_t)blockIdx.x * 64 >= cols) return;   // wave-uniform
  const int64_t h0 = s * kStepCodes;
  const bool full = vec && col0 + 4 <= cols;
  uint32_t r[64];   // byte c of r[h] = row h0 + h, column col0 + c (0 past the matrix)
#pragma unroll
  for (int h = 0; h < 64; ++h) {
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
    uint4 piece[12];
    pack_step([&](int h) { return byte_of(r[h], c, 255u); }, sh.lut, piece);
    wave_staged_store<12>(sh.stage[wave], sh.dsts[wave], piece,
                          col0 + c < cols ? out + (col0 + c) * ld_line + s * kStepBytes
                                          : nullptr);
  }
}

__device__ __forceinline__ v16f mfma_fp4(const v4i& a, const v4i& b, const v16f& c) {
  const v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  // cbsz = blgp = 4: both operands e2m1; scales 0x80 = 2^1 (E8M0) on both sides.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, 0x80, 0, 0x80);
}

// ------------------------------------------------------------------ 6 products (test path)
// One wave per 32 x 32 output block; fragments straight from global memory: lane (row =
// lane & 31, half = lane >> 5) supplies the 16 bytes (32 codes) at byte 32 t + 16 half of
// K step s of its line, identically for A and B.
__global__ __launch_bounds__(64) void awe_products_kernel(
    int64_t m, int64_t n, int64_t steps, const uint8_t* __restrict__ pa, int64_t lda,
    const uint8_t* __restrict__ pb, int64_t ldb, int32_t* __restrict__ out, int64_t ldo,
    int64_t stride_o) {
  const int lane = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.y * 32, col0 = (int64_t)blockIdx.x * 32;
  int64_t ra = row0 + (lane & 31), rb = col0 + (lane & 31);
  ra = ra < m ? ra : m - 1;
  rb = rb < n ? rb : n - 1;
  const int half = lane >> 5;
  v16f acc[kPlanes];
#pragma unroll
  for (int t = 0; t < kPlanes; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.0f;
  for (int64_t s = 0; s < steps; ++s) {
#pragma unroll
    for (int t = 0; t < kPlanes; ++t) {
      const int64_t off = s * kStepBytes + 32 * t + 16 * half;
      const v4i fa = *reinterpret_cast<const v4i*>(pa + ra * lda + off);
      const v4i fb = *reinterpret_cast<const v4i*>(pb + rb * ldb + off);
      acc[t] = mfma_fp4(fa, fb, acc[t]);
    }
  }
  const int64_t col = col0 + (lane & 31);
  if (col >= n) return;
#pragma unroll
  for (int t = 0; t < kPlanes; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = row0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (row < m) out[t * stride_o + row * ldo + col] = (int32_t)acc[t][v];
    }
}

// ------------------------------------------------------------------ fused weighted GEMM
// Workgroup tile 128 x 128, 512 threads = 8 waves.  Waves 2g and 2g+1 share the 64 x 64
// region g (rows 64 (g >> 1), columns 64 (g & 1)) and split the six products: wave 2g+h
// takes products 3h .. 3h+2, over 2 x 2 MFMA blocks of 32 x 32 (3 x 4 fp32 accumulators of
// 16 registers).  Per K step (64 codes) the tile needs 128 A lines and 128 B lines of 192
// bytes (48 KiB), loaded straight into a 3-stage LDS ring by global_load_lds_dwordx4 from
// wave-uniform SGPR bases plus fixed lane offsets (6 loads of 1 KiB per wave and step).
// LDS rows are 192 bytes: 12 chunks of 16 bytes, rotated by (row >> 2) & 3, so that the 16
// lanes of a fragment read (16 consecutive rows, one logical chunk) cover all 64 banks.
//
// Step t of a wave: the 4 MFMAs of its first product, reading the second product's four
// fragments between them; the second product's, reading the third's; a wait for its loads
// of step t+1 and its reads; the workgroup barrier (step t+1 complete in LDS, step t read by
// every wave); the third product's MFMAs, reading step t+1's first fragments and issuing
// its 6 loads of step t+3 into the stage of step t.  Past the last step the last step is
// loaded again.  Epilogue: each wave sums coef_t x (int) acc_t over its products in
// wrap-around 32-bit integers; the odd wave of each pair hands its partial sums to the
// even one through LDS, which adds them and stores C.
constexpr int AM = 128, AN = 128;
constexpr int kAweThreads = 512;
constexpr int kRowBytes = kStepBytes;               // 192
constexpr int kAweStage = (AM + AN) * kRowBytes;    // 48 KiB
constexpr int kAweStages = 3;
constexpr int kAweLoads = kAweStage / 1024 / 8;     // 6 per wave and step
constexpr int kAweGroupM = 4;
constexpr int kAweXcds = 8;
static_assert(kAweStages * kAweStage <= 160 * 1024, "ring fits the LDS");
static_assert(4 * 64 * 64 * 4 <= kAweStages * kAweStage, "epilogue exchange fits the ring");

// Workgroup barrier that is also a compiler barrier for memory operations, so that no
// LDS access moves across it.
__device__ __forceinline__ void awe_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kAweThreads, 1) void awe_gemm_kernel(
    int64_t m, int64_t n, int64_t steps, const uint8_t* __restrict__ pa, int64_t lda,
    const uint8_t* __restrict__ pb, int64_t ldb, int32_t* __restrict__ c, int64_t ldc,
    int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kAweStages * kAweStage];

  // Block -> tile: XCD-contiguous, then grouped by kAweGroupM tile rows.
  const int total = gridDim.x;
  int bid = blockIdx.x;
  if (total % kAweXcds == 0) bid = (bid % kAweXcds) * (total / kAweXcds) + bid / kAweXcds;
  const int per_group = kAweGroupM * tiles_n;
  const int first_m = (bid / per_group) * kAweGroupM;
  const int gsize = tiles_m - first_m < kAweGroupM ? tiles_m - first_m : kAweGroupM;
  const int in_group = bid % per_group;
  const int64_t row0 = (int64_t)(first_m + in_group % gsize) * AM;
  const int64_t col0 = (int64_t)(in_group / gsize) * AN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 1;          // region
  const int h = wave & 1;           // products 3h .. 3h+2
  const int r0 = (g >> 1) * 64;     // region rows within the tile
  const int c0 = (g & 1) * 64;      // region columns

  // Direct loads: load q of this wave covers stage bytes 1024 (wave + 8 q) .. +1023; lane
  // i writes byte b = 1024 (wave + 8 q) + 16 i, which is LDS row b / 192, physical chunk
  // (b % 192) / 16, holding logical chunk (physical - rotation) mod 12 of that row's K
  // step.  Rows 0..127 are A lines row0.., rows 128..255 B lines col0.. (q < 3: A).
  // Lines past the matrix re-read its last line.
  uint32_t voff[kAweLoads];
#pragma unroll
  for (int q = 0; q < kAweLoads; ++q) {
    const int b = 1024 * (wave + 8 * q) + 16 * lane;
    const int row = b / kRowBytes;
    const int pc = (b % kRowBytes) >> 4;
    int lc = pc - ((row >> 2) & 3);
    lc = lc < 0 ? lc + 12 : lc;
    const bool is_b = q >= kAweLoads / 2;
    const int64_t origin = is_b ? col0 : row0;
    const int64_t last = (is_b ? n : m) - 1;
    const int64_t line = origin + (row & 127) < last ? origin + (row & 127) : last;
    voff[q] = (uint32_t)((line - origin) * (is_b ? ldb : lda) + 16 * lc);
  }
  const uint64_t base_a = (uint64_t)(pa + row0 * lda), base_b = (uint64_t)(pb + col0 * ldb);
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(lds_address(lds) + wave * 1024);
  const int nk = (int)steps;
  auto issue = [&](int q, int tk, int stage) {
    const uint64_t kb = (uint64_t)tk * kStepBytes;
    const uint32_t dst = wave_lds + (uint32_t)stage * kAweStage + q * (8 * 1024);
    dma16_sbase(voff[q], (q < kAweLoads / 2 ? base_a : base_b) + kb, dst);
  };

  v16f acc[3][2][2];
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[p][i][j][v] = 0.0f;

  // Fragment reads: lane (row = lane & 31, half = lane >> 5) of a 32-row block, logical
  // chunk 2 t + half of its row (plane t, codes 32 half .. 32 half + 31 of the step).  All
  // fragment rows of a lane share row mod 16 = lane mod 16, hence one rotation.
  const int frow = lane & 31, fhalf = lane >> 5;
  const int rot = (frow >> 2) & 3;
  int offa[2], offb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) offa[i] = (r0 + 32 * i + frow) * kRowBytes;
#pragma unroll
  for (int j = 0; j < 2; ++j) offb[j] = (AM + c0 + 32 * j + frow) * kRowBytes;
  int chunk_off[3];   // byte offset of this lane's chunk of each of its products
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    int pc = 2 * (3 * h + p) + fhalf + rot;
    pc = pc < 12 ? pc : pc - 12;
    chunk_off[p] = pc << 4;
  }
  // frag[set][0..1] = A blocks, [2..3] = B blocks
  v4i frag[2][4];
  auto read = [&](int set, int stage, int p, int idx) {
    const uint8_t* st = lds + stage * kAweStage + chunk_off[p];
    const int off = idx < 2 ? offa[idx] : offb[idx - 2];
    frag[set][idx] = *reinterpret_cast<const v4i*>(st + off);
  };
  // the 4 MFMAs of product p from fragment set `set`, the reads of (rp, rstage) into the
  // other set between them, and loads [l0, l1) of step lt into stage ls after MFMAs.
  auto product = [&](int set, int p, int rp, int rstage, bool do_read, int l0, int l1, int lt,
                     int ls) {
#pragma unroll
    for (int idx = 0; idx < 4; ++idx) {
      const int i = idx >> 1, j = idx & 1;
      acc[p][i][j] = mfma_fp4(frag[set][i], frag[set][2 + j], acc[p][i][j]);
      if (do_read) read(set ^ 1, rstage, rp, idx);
      const int qa = l0 + 2 * idx, qb = qa + 1;
      if (qa < l1) issue(qa, lt, ls);
      if (qb < l1) issue(qb, lt, ls);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int q = 0; q < kAweLoads; ++q) issue(q, s < nk ? s : nk - 1, s);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kAweLoads) : "memory");  // step 0 landed
  awe_barrier();
#pragma unroll
  for (int idx = 0; idx < 4; ++idx) read(0, 0, 0, idx);

  // One step with the first product's fragments in set `s0`; parity alternates because
  // three products per step flip the set three times.
  auto step = [&](int t, int s0) {
    const int st = t % kAweStages;
    __builtin_amdgcn_sched_barrier(0);
    product(s0, 0, 1, st, true, 0, 0, 0, 0);
    product(s0 ^ 1, 1, 2, st, true, 0, 0, 0, 0);
    // step t+1 landed (this wave's loads; the barrier covers the others), step t+2's
    // loads may still be in flight; every read of step t is done
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kAweLoads) : "memory");
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    awe_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int tn = t + 1 < nk ? t + 1 : t;       // past the last step: a harmless re-read
    const int tl = t + 3 < nk ? t + 3 : nk - 1;  // past the last step: reload the last
    product(s0, 2, 0, tn % kAweStages, true, 0, kAweLoads, tl, st);
  };
  int t = 0;
  for (; t + 1 < nk; t += 2) {
    step(t, 0);
    step(t + 1, 1);
  }
  if (t < nk) step(t, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  awe_barrier();   // every wave is past its last load and LDS read of the ring

  // Epilogue: weighted sum of this wave's products, the odd wave's through LDS.
  uint32_t part[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        uint32_t sum = 0;
#pragma unroll
        for (int p = 0; p < 3; ++p)
          sum += (uint32_t)kCoef[3 * h + p] * (uint32_t)(int32_t)acc[p][i][j][v];
        part[i][j][v] = sum;
      }
  uint32_t* xch = reinterpret_cast<uint32_t*>(lds) + g * (4 * 16 * 64);
  if (h == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) xch[((2 * i + j) * 16 + v) * 64 + lane] = part[i][j][v];
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  awe_barrier();
  if (h == 1) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = col0 + c0 + 32 * j + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t sum = part[i][j][v] + xch[((2 * i + j) * 16 + v) * 64 + lane];
        const int64_t row = row0 + r0 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < m && col < n) c[row * ldc + col] = (int32_t)sum;
      }
    }
}

}  // namespace

int64_t awe_line_bytes(int64_t k) { return round_up(k, kStepCodes) / kStepCodes * kStepBytes; }

int launch_awe_pack(const int8_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                    uint8_t* out, int64_t ld_line, hipStream_t s) {
  const int64_t kdim = axis == 0 ? cols : rows;
  const int64_t steps = round_up(kdim, kStepCodes) / kStepCodes;
  if (axis == 0) {
    if (rows <= 0 || steps <= 0) return OZK_OK;
    const int64_t threads = rows * steps;
    const int vec = (reinterpret_cast<uintptr_t>(x) % 16) == 0 && ldx % 16 == 0;
    hipLaunchKernelGGL(awe_pack_rows_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                       0, s, x, rows, cols, ldx, out, ld_line, steps, vec);
  } else {
    if (cols <= 0 || steps <= 0) return OZK_OK;
    const int vec = (reinterpret_cast<uintptr_t>(x) % 4) == 0 && ldx % 4 == 0;
    dim3 grid((unsigned)((cols + 255) / 256), (unsigned)((steps + 3) / 4));
    hipLaunchKernelGGL(awe_pack_cols_kernel, grid, dim3(256), 0, s, x, rows, cols, ldx, out,
                       ld_line, steps, vec);
  }
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

int launch_awe_products(int64_t m, int64_t n, int64_t steps, const uint8_t* pa, int64_t lda,
                        const uint8_t* pb, int64_t ldb, int32_t* out, int64_t ldo,
                        int64_t stride_o, hipStream_t s) {
  if (m <= 0 || n <= 0) return OZK_OK;
  dim3 grid((unsigned)((n + 31) / 32), (unsigned)((m + 31) / 32));
  hipLaunchKernelGGL(awe_products_kernel, grid, dim3(64), 0, s, m, n, steps, pa, lda, pb, ldb,
                     out, ldo, stride_o);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

int launch_awe_gemm(int64_t m, int64_t n, int64_t steps, const uint8_t* pa, int64_t lda,
                    const uint8_t* pb, int64_t ldb, int32_t* c, int64_t ldc, hipStream_t s) {
  if (m <= 0 || n <= 0) return OZK_OK;
  // 32-bit lane offsets within a 128-line tile; line strides hold every step
  if (steps <= 0 || lda < steps * kStepBytes || ldb < steps * kStepBytes || lda % 16 ||
      ldb % 16 || 128 * (lda > ldb ? lda : ldb) >= ((int64_t)1 << 31))
    return OZK_EINVAL;
  const int64_t tiles_m = (m + AM - 1) / AM, tiles_n = (n + AN - 1) / AN;
  if (tiles_m * tiles_n > 0x7fffffff) return OZK_EUNSUPPORTED;
  hipLaunchKernelGGL(awe_gemm_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kAweThreads), 0,
                     s, m, n, steps, pa, lda, pb, ldb, c, ldc, (int)tiles_m, (int)tiles_n);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

}  // namespace ozk
