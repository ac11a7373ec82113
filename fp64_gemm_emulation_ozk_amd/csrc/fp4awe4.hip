// Exact INT4 x INT8 matrix products in 4 FP4 products on the gfx950 scaled f8f6f4 MFMA.
// [AWE] (arXiv 2609.24519 listing, English abstract): with free integer limb weights and
// stored planes that are linear combinations of limbs, an INT4 x INT8 product takes 4 FP4
// matrix products.
//
// Encoding: an int4 x = a0 + 5 a1 and an int8 y = b0 + 5 b1 + 25 b2 are the values at
// (5, 1) of the binary forms X(p, q) = q a0 + p a1 and Y(p, q) = q^2 b0 + p q b1 + p^2 b2,
// so x y is the value at (5, 1) of the cubic form X Y.  Its four coefficients follow from
// X Y at the points (p, q) = (0, 1), (1, 0), (1, 1), (1, 2); the stored planes are X and Y
// there:
//     U = (a0, a1, a0 + a1, 2 a0 + a1),     V = (b0, b2, b0 + b1 + b2, 4 b0 + 2 b1 + b2),
// every one of them in S = 2 x FP4 = {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12} (b1 is not
// stored).  Interpolating and evaluating at (5, 1) gives
//     x y = 36 U_0 V_0 + 90 U_1 V_1 + 45 U_2 V_2 - 10 U_3 V_3,
// so C = A B = sum_t coef_t U_t(A) V_t(B): four plane products.  Of the limb tuples that
// encode a value, the one with the smallest largest plane magnitude, then the smallest sum
// of squares of its planes, then the smallest limbs lexicographically; the A planes are
// then at most 4 and the B planes at most 12 in magnitude, so every elementary product is
// at most 48 and fp32 sums are exact for K <= 349525.  The weighted sum is taken in
// wrap-around 32-bit integers (the exact result fits int32).  An int4 value is the low
// four bits of its byte (two's complement).
//
// Each plane product is an e2m1 x e2m1 MFMA with both E8M0 block scales 2^1 (plane value
// d stored as the code of d/2).  Layout of the packed planes (per line: a row of A, a
// column of B): K in steps of 64 codes; step s of line i occupies bytes 128 s .. 128 s +
// 127, plane t at byte 32 t of the step, two codes per byte with the even K index in the
// low nibble.  A K step of a 128-line tile is then 128 contiguous cache lines.
#include <type_traits>

#include "fp4_pack.h"
#include "lds_dma.h"
#include "ozk_internal.h"

namespace ozk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWeight = 5;
constexpr int kPlanes4 = 4;
constexpr int kStepCodes4 = 64;
constexpr int kStepBytes4 = kPlanes4 * kStepCodes4 / 2;   // 128
constexpr int kCoef4[kPlanes4] = {36, 90, 45, -10};

// ------------------------------------------------------------------ encoding tables
constexpr int twice_e2m1_4(int code) {  // 2 x the value of an e2m1 code: an integer in S
  const int e = (code >> 1) & 3, mbit = code & 1;
  const int mag = e == 0 ? mbit : (1 << e) + (mbit << (e - 1));
  return (code & 8) ? -mag : mag;
}

struct CodeOf4 {
  int c[49];   // c[d + 24]: the e2m1 code of d/2 (+0 for 0), -1 where d is not in S
};
constexpr CodeOf4 make_code_of4() {
  CodeOf4 t{};
  for (int d = 0; d < 49; ++d) t.c[d] = -1;
  for (int code = 15; code >= 0; --code) t.c[twice_e2m1_4(code) + 24] = code;  // +0 last
  return t;
}
constexpr CodeOf4 kCodeOf4 = make_code_of4();
constexpr int code4(int d) { return d < -24 || d > 24 ? -1 : kCodeOf4.c[d + 24]; }
constexpr int iabs4(int v) { return v < 0 ? -v : v; }

// Lexicographic "less" on (largest magnitude, sum of squares, limbs...).
template <int N>
constexpr bool key_less(const int (&a)[N], const int (&b)[N]) {
  for (int i = 0; i < N; ++i)
    if (a[i] != b[i]) return a[i] < b[i];
  return false;
}

struct Awe4Tables {
  uint16_t x_codes[16];    // index x + 8: code of plane t in bits 4t .. 4t + 3
  uint16_t y_codes[256];   // index y + 128
};

// The limbs that are planes themselves (a0, a1 of x; b0, b2 of y) range over S; the
// remaining limb b1 follows from y, and the other planes must land in S as well.
constexpr Awe4Tables make_awe4_tables() {
  Awe4Tables t{};
  for (int x = -8; x < 8; ++x) {
    int best[4] = {1 << 20, 0, 0, 0};
    int planes[4] = {0, 0, 0, 0};
    for (int c1 = 0; c1 < 16; ++c1) {
      if (c1 == 8) continue;   // -0: the same value as code 0
      const int a1 = twice_e2m1_4(c1), a0 = x - kWeight * a1;
      const int u[4] = {a0, a1, a0 + a1, 2 * a0 + a1};
      bool ok = true;
      int mx = 0, sq = 0;
      for (int q = 0; q < 4; ++q) {
        ok = ok && code4(u[q]) >= 0;
        mx = iabs4(u[q]) > mx ? iabs4(u[q]) : mx;
        sq += u[q] * u[q];
      }
      const int key[4] = {mx, sq, a0, a1};
      if (ok && key_less(key, best)) {
        for (int q = 0; q < 4; ++q) best[q] = key[q], planes[q] = u[q];
      }
    }
    uint16_t w = 0;
    for (int q = 0; q < 4; ++q) w |= (uint16_t)(code4(planes[q]) << (4 * q));
    t.x_codes[x + 8] = w;
  }
  for (int y = -128; y < 128; ++y) {
    int best[5] = {1 << 20, 0, 0, 0, 0};
    int planes[4] = {0, 0, 0, 0};
    for (int c0 = 0; c0 < 16; ++c0) {
      if (c0 == 8) continue;
      for (int c2 = 0; c2 < 16; ++c2) {
        if (c2 == 8) continue;
        const int b0 = twice_e2m1_4(c0), b2 = twice_e2m1_4(c2);
        const int rest = y - b0 - kWeight * kWeight * b2;
        if (rest % kWeight != 0) continue;
        const int b1 = rest / kWeight;
        const int v[4] = {b0, b2, b0 + b1 + b2, 4 * b0 + 2 * b1 + b2};
        bool ok = true;
        int mx = 0, sq = 0;
        for (int q = 0; q < 4; ++q) {
          ok = ok && code4(v[q]) >= 0;
          mx = iabs4(v[q]) > mx ? iabs4(v[q]) : mx;
          sq += v[q] * v[q];
        }
        const int key[5] = {mx, sq, b0, b1, b2};
        if (ok && key_less(key, best)) {
          for (int q = 0; q < 5; ++q) best[q] = key[q];
          for (int q = 0; q < 4; ++q) planes[q] = v[q];
        }
      }
    }
    uint16_t w = 0;
    for (int q = 0; q < 4; ++q) w |= (uint16_t)(code4(planes[q]) << (4 * q));
    t.y_codes[y + 128] = w;
  }
  return t;
}

__constant__ Awe4Tables d_awe4 = make_awe4_tables();
static_assert(make_awe4_tables().x_codes[8] == 0 && make_awe4_tables().y_codes[128] == 0,
              "0 encodes as four zero planes");

// ------------------------------------------------------------------ packers
// A packer's table in LDS: the spread word (byte t = code of plane t) of every value,
// indexed by the low nibble of the stored byte (int4, A side) or by the unsigned byte
// (int8, B side).
template <bool kInt4>
__device__ __forceinline__ void load_lut4(uint32_t* lut) {
  const int b = threadIdx.x;   // 256 threads
  if (kInt4) {
    if (b < 16) lut[b] = spread_nibbles(d_awe4.x_codes[b ^ 8]);
  } else {
    lut[b] = spread_nibbles(d_awe4.y_codes[b ^ 0x80]);
  }
  __syncthreads();
}

// 64 consecutive K values of one line -> the 128 bytes of its K step as 8 pieces of 16
// (piece 2 t + half: plane t, values 32 half .. 32 half + 31); at(h) is the table index
// of value h.
template <typename At>
__device__ __forceinline__ void pack_step4(At at, const uint32_t* lut, uint4 (&piece)[8]) {
  uint32_t w[kPlanes4][8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t sw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) sw[u] = lut[at(8 * q + u)];
    uint32_t o[kPlanes4];
    pack8_planes<kPlanes4>(sw, o);
#pragma unroll
    for (int t = 0; t < kPlanes4; ++t) w[t][q] = o[t];
  }
#pragma unroll
  for (int t = 0; t < kPlanes4; ++t) {
    piece[2 * t] = make_uint4(w[t][0], w[t][1], w[t][2], w[t][3]);
    piece[2 * t + 1] = make_uint4(w[t][4], w[t][5], w[t][6], w[t][7]);
  }
}

// Per-block LDS of the packers: the table and, per wave, 64 staged K steps and their
// destinations.
struct Awe4PackShared {
  uint32_t lut[256];
  uint4 stage[4][64 * 8];
  uint8_t* dsts[4][64];
};

// axis 0: x rows x cols (K = cols); thread -> (row, K step); consecutive threads take
// consecutive steps of a row, so the staged stores of a wave write 8 KiB runs.  vec: x and
// ldx 16-byte aligned, so a whole step of 64 values is four 16-byte loads.
template <bool kInt4>
__global__ __launch_bounds__(256) void awe4_pack_rows_kernel(const int8_t* __restrict__ x,
                                                             int64_t rows, int64_t cols,
                                                             int64_t ldx, uint8_t* __restrict__ out,
                                                             int64_t ld_line, int64_t steps,
                                                             int vec) {
  __shared__ Awe4PackShared sh;
  load_lut4<kInt4>(sh.lut);
  const int wave = threadIdx.x >> 6;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t wave_g0 = g - (threadIdx.x & 63);
  if (wave_g0 >= rows * steps) return;            // the whole wave is past the end
  const bool valid = g < rows * steps;
  const int64_t gg = valid ? g : wave_g0;           // lanes past the end pack a copy
  const int64_t row = gg / steps;
  const int64_t s = gg - row * steps;
  const int64_t h0 = s * kStepCodes4;
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
  constexpr uint32_t mask = kInt4 ? 15u : 255u;
  uint4 piece[8];
  pack_step4([&](int h) { return byte_of(d[h >> 2], h & 3, mask); }, sh.lut, piece);
  wave_staged_store<8>(sh.stage[wave], sh.dsts[wave], piece,
                       valid ? out + row * ld_line + s * kStepBytes4 : nullptr);
}

// axis 1: x rows x cols with K = rows; thread -> (4 consecutive columns, K step).  The 64
// threads of a wave take 256 consecutive columns, so with vec (x and ldx 4-byte aligned)
// every load instruction reads 256 consecutive bytes of one row; each of the 4 column
// rounds stores whole 128-byte steps through the staging area.
template <bool kInt4>
__global__ __launch_bounds__(256) void awe4_pack_cols_kernel(const int8_t* __restrict__ x,
                                                             int64_t rows, int64_t cols,
                                                             int64_t ldx, uint8_t* __restrict__ out,
                                                             int64_t ld_line, int64_t steps,
                                                             int vec) {
  __shared__ Awe4PackShared sh;
  load_lut4<kInt4>(sh.lut);
  const int wave = threadIdx.x >> 6;
  const int64_t col0 = 4 * ((int64_t)blockIdx.x * 64 + (threadIdx.x & 63));
  const int64_t s = (int64_t)blockIdx.y * 4 + wave;
  if (s >= steps || 4 * (int64_t)blockIdx.x * 64 >= cols) return;   // wave-uniform
  const int64_t h0 = s * kStepCodes4;
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
  constexpr uint32_t mask = kInt4 ? 15u : 255u;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 piece[8];
    pack_step4([&](int h) { return byte_of(r[h], c, mask); }, sh.lut, piece);
    wave_staged_store<8>(sh.stage[wave], sh.dsts[wave], piece,
                         col0 + c < cols ? out + (col0 + c) * ld_line + s * kStepBytes4
                                         : nullptr);
  }
}

__device__ __forceinline__ v16f mfma_fp4_32(const v4i& a, const v4i& b, const v16f& c) {
  const v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  // cbsz = blgp = 4: both operands e2m1; scales 0x80 = 2^1 (E8M0) on both sides.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, 0x80, 0, 0x80);
}

// ------------------------------------------------------------------ 4 products (test path)
// One wave per 32 x 32 output block; fragments straight from global memory: lane (row =
// lane & 31, half = lane >> 5) supplies the 16 bytes (32 codes) at byte 32 t + 16 half of
// K step s of its line, identically for A and B.
__global__ __launch_bounds__(64) void awe4_products_kernel(
    int64_t m, int64_t n, int64_t steps, const uint8_t* __restrict__ pa, int64_t lda,
    const uint8_t* __restrict__ pb, int64_t ldb, int32_t* __restrict__ out, int64_t ldo,
    int64_t stride_o) {
  const int lane = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.y * 32, col0 = (int64_t)blockIdx.x * 32;
  int64_t ra = row0 + (lane & 31), rb = col0 + (lane & 31);
  ra = ra < m ? ra : m - 1;
  rb = rb < n ? rb : n - 1;
  const int half = lane >> 5;
  v16f acc[kPlanes4];
#pragma unroll
  for (int t = 0; t < kPlanes4; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.0f;
  for (int64_t s = 0; s < steps; ++s) {
#pragma unroll
    for (int t = 0; t < kPlanes4; ++t) {
      const int64_t off = s * kStepBytes4 + 32 * t + 16 * half;
      const v4i fa = *reinterpret_cast<const v4i*>(pa + ra * lda + off);
      const v4i fb = *reinterpret_cast<const v4i*>(pb + rb * ldb + off);
      acc[t] = mfma_fp4_32(fa, fb, acc[t]);
    }
  }
  const int64_t col = col0 + (lane & 31);
  if (col >= n) return;
#pragma unroll
  for (int t = 0; t < kPlanes4; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = row0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (row < m) out[t * stride_o + row * ldo + col] = (int32_t)acc[t][v];
    }
}

// ------------------------------------------------------------------ fused weighted GEMM
// Products 1 and 2 share an accumulator: with block scales 2^2 x 2^1 on product 1 (twice
// the 2^1 x 2^1 of the others) it adds 2 P1 + P2, and C = 36 P0 + 45 (2 P1 + P2) - 10 P3.
// Per K value |2 u1 v1 + u2 v2| <= 27 over all int4 x int8 pairs (|u0 v0| <= 18,
// |u3 v3| <= 48), so all three fp32 sums stay exact integers for K <= 349525.
//
// Workgroup tile 128 x 256, 512 threads = 8 waves; wave w computes all four products of
// the 64 x 64 region (rows 64 (w >> 2), columns 64 (w & 3)) as 2 x 2 blocks of 32 x 32 in
// three accumulator sets (192 registers).  Three sets per output, instead of one per
// product, are what let the tile grow from 128 x 128: per K step (64 codes) it needs 128
// A lines and 256 B lines of 128 bytes (48 KiB) for 128 MFMAs, 384 bytes per MFMA instead
// of 512.  The lines go straight into a 3-stage LDS ring by global_load_lds_dwordx4 from
// wave-uniform SGPR bases plus fixed lane offsets (6 loads of 1 KiB per wave and step).
// LDS rows are 128 bytes: 8 chunks of 16 bytes, XOR-swizzled by (row >> 1) & 7, so that
// the 16 lanes of a fragment read (16 consecutive rows, one logical chunk) cover all 64
// banks.
//
// Step t of a wave: products 0, 1 and 2 (4 MFMAs each), each reading the next product's
// four fragments between its MFMAs; a wait for its loads of step t+1 and its reads; the
// workgroup barrier (step t+1 complete in LDS, step t read by every wave); product 3,
// reading step t+1's product-0 fragments and issuing its 6 loads of step t+3 into the
// stage of step t.  Past the last step the last step is loaded again.  Epilogue: each
// lane combines its three sums in wrap-around 32-bit integers and stores C.
constexpr int BM4 = 128, BN4 = 256;
constexpr int kAwe4Threads = 512;
constexpr int kRowBytes4 = kStepBytes4;                 // 128
constexpr int kAwe4Stage = (BM4 + BN4) * kRowBytes4;    // 48 KiB
constexpr int kAwe4Stages = 3;
constexpr int kAwe4Loads = kAwe4Stage / 1024 / 8;       // 6 per wave and step
// 8 tile rows per group: an XCD's 32 tiles in flight span 8 x 4 tiles, (8 x 128 + 4 x 256)
// lines per K step (4 x 8: 1.3 % slower at 8192^3, 2 x 16: 3.9 % slower)
constexpr int kAwe4GroupM = 8;
constexpr int kAwe4Xcds = 8;
static_assert(kAwe4Stages * kAwe4Stage <= 160 * 1024, "ring fits the LDS");
static_assert(kAwe4Loads == 6 && BM4 * kRowBytes4 == 2 * 8192, "A rows are loads 0 and 1");
static_assert(kCoef4[1] == 2 * kCoef4[2], "products 1 and 2 share a sum at scales 2 : 1");

__device__ __forceinline__ void awe4_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Product t's MFMA: block scales 2^1 on both operands (each code holds half its plane
// value), 2^2 on A for product 1 (added twice into the shared sum).
template <int kScaleA>
__device__ __forceinline__ v16f mfma_fp4_32s(const v4i& a, const v4i& b, const v16f& c) {
  const v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, kScaleA, 0, 0x80);
}

__global__ __launch_bounds__(kAwe4Threads, 1) void awe4_gemm_kernel(
    int64_t m, int64_t n, int64_t steps, const uint8_t* __restrict__ pa, int64_t lda,
    const uint8_t* __restrict__ pb, int64_t ldb, int32_t* __restrict__ c, int64_t ldc,
    int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kAwe4Stages * kAwe4Stage];

  // Block -> tile: XCD-contiguous, then grouped by kAwe4GroupM tile rows.
  const int total = gridDim.x;
  int bid = blockIdx.x;
  if (total % kAwe4Xcds == 0) bid = (bid % kAwe4Xcds) * (total / kAwe4Xcds) + bid / kAwe4Xcds;
  const int per_group = kAwe4GroupM * tiles_n;
  const int first_m = (bid / per_group) * kAwe4GroupM;
  const int gsize = tiles_m - first_m < kAwe4GroupM ? tiles_m - first_m : kAwe4GroupM;
  const int in_group = bid % per_group;
  const int64_t row0 = (int64_t)(first_m + in_group % gsize) * BM4;
  const int64_t col0 = (int64_t)(in_group / gsize) * BN4;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r0 = (wave >> 2) * 64;   // region rows within the tile
  const int c0 = (wave & 3) * 64;    // region columns

  // Direct loads: load q of this wave covers stage bytes 1024 (wave + 8 q) .. +1023, i.e.
  // LDS rows 8 (wave + 8 q) .. +7; lane i writes row 8 (wave + 8 q) + i / 8 at physical
  // chunk i % 8, which holds logical chunk (i % 8) ^ ((row >> 1) & 7) of that row's K step.
  // Rows 0..127 are A lines row0.. (q < 2), rows 128..383 B lines col0..; lines past the
  // matrix re-read its last line.
  uint32_t voff[kAwe4Loads];
#pragma unroll
  for (int q = 0; q < kAwe4Loads; ++q) {
    const int row = 8 * (wave + 8 * q) + (lane >> 3);
    const int lc = (lane & 7) ^ ((row >> 1) & 7);
    const bool is_b = q >= 2;
    const int64_t origin = is_b ? col0 : row0;
    const int64_t last = (is_b ? n : m) - 1;
    const int rel = is_b ? row - BM4 : row;
    const int64_t line = origin + rel < last ? origin + rel : last;
    voff[q] = (uint32_t)((line - origin) * (is_b ? ldb : lda) + 16 * lc);
  }
  const uint64_t base_a = (uint64_t)(pa + row0 * lda), base_b = (uint64_t)(pb + col0 * ldb);
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(lds_address(lds) + wave * 1024);
  const int nk = (int)steps;
  auto issue = [&](int q, int tk, int stage) {
    const uint64_t kb = (uint64_t)tk * kStepBytes4;
    const uint32_t dst = wave_lds + (uint32_t)stage * kAwe4Stage + q * (8 * 1024);
    dma16_sbase(voff[q], (q < 2 ? base_a : base_b) + kb, dst);
  };

  v16f acc[3][2][2];   // sums of P0, 2 P1 + P2, P3
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
  // fragment rows of a lane share (row >> 1) & 7 = (lane >> 1) & 7, hence one swizzle.
  const int frow = lane & 31, fhalf = lane >> 5;
  const int sw = (frow >> 1) & 7;
  int offa[2], offb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) offa[i] = (r0 + 32 * i + frow) * kRowBytes4;
#pragma unroll
  for (int j = 0; j < 2; ++j) offb[j] = (BM4 + c0 + 32 * j + frow) * kRowBytes4;
  int chunk_off[kPlanes4];   // byte offset of this lane's chunk of each plane
#pragma unroll
  for (int t = 0; t < kPlanes4; ++t) chunk_off[t] = ((2 * t + fhalf) ^ sw) << 4;
  // frag[set][0..1] = A blocks, [2..3] = B blocks
  v4i frag[2][4];
  auto read = [&](int set, int stage, int t, int idx) {
    const uint8_t* st = lds + stage * kAwe4Stage + chunk_off[t];
    const int off = idx < 2 ? offa[idx] : offb[idx - 2];
    frag[set][idx] = *reinterpret_cast<const v4i*>(st + off);
  };
  // the 4 MFMAs of product t (into sum a, A scale kScaleA) from fragment set `set`, the
  // reads of plane rt of stage rstage into the other set between them, and loads [0, nl)
  // of step lt into stage ls, two per MFMA.
  auto product = [&](auto scale_a, int set, int a, int rt, int rstage, int nl, int lt, int ls) {
#pragma unroll
    for (int idx = 0; idx < 4; ++idx) {
      const int i = idx >> 1, j = idx & 1;
      acc[a][i][j] = mfma_fp4_32s<decltype(scale_a)::value>(frag[set][i], frag[set][2 + j],
                                                             acc[a][i][j]);
      read(set ^ 1, rstage, rt, idx);
      if (2 * idx < nl) issue(2 * idx, lt, ls);
      if (2 * idx + 1 < nl) issue(2 * idx + 1, lt, ls);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using S1 = std::integral_constant<int, 0x80>;
  using S2 = std::integral_constant<int, 0x81>;

#pragma unroll
  for (int s = 0; s < kAwe4Stages; ++s)
#pragma unroll
    for (int q = 0; q < kAwe4Loads; ++q) issue(q, s < nk ? s : nk - 1, s);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kAwe4Stages - 1) * kAwe4Loads) : "memory");  // step 0
  awe4_barrier();
#pragma unroll
  for (int idx = 0; idx < 4; ++idx) read(0, 0, 0, idx);

  for (int t = 0; t < nk; ++t) {
    const int st = t % kAwe4Stages;
    __builtin_amdgcn_sched_barrier(0);
    product(S1{}, 0, 0, 1, st, 0, 0, 0);   // P0, reading P1
    product(S2{}, 1, 1, 2, st, 0, 0, 0);   // 2 P1, reading P2
    product(S1{}, 0, 1, 3, st, 0, 0, 0);   // P2, reading P3
    // step t+1 landed (this wave's loads; the barrier covers the others), step t+2's
    // loads may still be in flight; every read of step t is done
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kAwe4Stages - 2) * kAwe4Loads) : "memory");
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    awe4_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int tn = t + 1 < nk ? t + 1 : t;       // past the last step: a harmless re-read
    // past the last step: reload the last
    const int tl = t + kAwe4Stages < nk ? t + kAwe4Stages : nk - 1;
    product(S1{}, 1, 2, 0, tn % kAwe4Stages, kAwe4Loads, tl, st);   // P3, reading next P0
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = col0 + c0 + 32 * j + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t sum = (uint32_t)kCoef4[0] * (uint32_t)(int32_t)acc[0][i][j][v] +
                             (uint32_t)kCoef4[2] * (uint32_t)(int32_t)acc[1][i][j][v] +
                             (uint32_t)kCoef4[3] * (uint32_t)(int32_t)acc[2][i][j][v];
        const int64_t row = row0 + r0 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < m && col < n) c[row * ldc + col] = (int32_t)sum;
      }
    }
}

}  // namespace

int64_t awe4_line_bytes(int64_t k) {
  return round_up(k, kStepCodes4) / kStepCodes4 * kStepBytes4;
}

int launch_awe4_pack(const int8_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                     int int4, uint8_t* out, int64_t ld_line, hipStream_t s) {
  const int64_t kdim = axis == 0 ? cols : rows;
  const int64_t steps = round_up(kdim, kStepCodes4) / kStepCodes4;
  if (axis == 0) {
    if (rows <= 0 || steps <= 0) return OZK_OK;
    const int64_t threads = rows * steps;
    const int vec = (reinterpret_cast<uintptr_t>(x) % 16) == 0 && ldx % 16 == 0;
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (int4)
      hipLaunchKernelGGL(awe4_pack_rows_kernel<true>, grid, dim3(256), 0, s, x, rows, cols, ldx,
                         out, ld_line, steps, vec);
    else
      hipLaunchKernelGGL(awe4_pack_rows_kernel<false>, grid, dim3(256), 0, s, x, rows, cols, ldx,
                         out, ld_line, steps, vec);
  } else {
    if (cols <= 0 || steps <= 0) return OZK_OK;
    const int vec = (reinterpret_cast<uintptr_t>(x) % 4) == 0 && ldx % 4 == 0;
    const dim3 grid((unsigned)((cols + 255) / 256), (unsigned)((steps + 3) / 4));
    if (int4)
      hipLaunchKernelGGL(awe4_pack_cols_kernel<true>, grid, dim3(256), 0, s, x, rows, cols, ldx,
                         out, ld_line, steps, vec);
    else
      hipLaunchKernelGGL(awe4_pack_cols_kernel<false>, grid, dim3(256), 0, s, x, rows, cols, ldx,
                         out, ld_line, steps, vec);
  }
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

int launch_awe4_products(int64_t m, int64_t n, int64_t steps, const uint8_t* pa, int64_t lda,
                         const uint8_t* pb, int64_t ldb, int32_t* out, int64_t ldo,
                         int64_t stride_o, hipStream_t s) {
  if (m <= 0 || n <= 0) return OZK_OK;
  dim3 grid((unsigned)((n + 31) / 32), (unsigned)((m + 31) / 32));
  hipLaunchKernelGGL(awe4_products_kernel, grid, dim3(64), 0, s, m, n, steps, pa, lda, pb, ldb,
                     out, ldo, stride_o);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

int launch_awe4_gemm(int64_t m, int64_t n, int64_t steps, const uint8_t* pa, int64_t lda,
                     const uint8_t* pb, int64_t ldb, int32_t* c, int64_t ldc, hipStream_t s) {
  if (m <= 0 || n <= 0) return OZK_OK;
  // 32-bit lane offsets within a 256-line tile; line strides hold every step
  if (steps <= 0 || lda < steps * kStepBytes4 || ldb < steps * kStepBytes4 || lda % 16 ||
      ldb % 16 || BN4 * (lda > ldb ? lda : ldb) >= ((int64_t)1 << 31))
    return OZK_EINVAL;
  const int64_t tiles_m = (m + BM4 - 1) / BM4, tiles_n = (n + BN4 - 1) / BN4;
  if (tiles_m * tiles_n > 0x7fffffff) return OZK_EUNSUPPORTED;
  hipLaunchKernelGGL(awe4_gemm_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kAwe4Threads),
                     0, s, m, n, steps, pa, lda, pb, ldb, c, ldc, (int)tiles_m, (int)tiles_n);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

}  // namespace ozk
