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
// Products: v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in e2m1 and both E8M0
// block scales equal to 2^1, so every elementary product is the integer d_a d_b.  The 9
// digit products are summed per weight class w = da + db (5 fp32 accumulators).  Each
// K element adds at most 128 in magnitude to any class (class 1: |d0 d1| + |d1 d0|), so
// for K <= 131071 every partial sum is an integer below 2^24 and fp32 holds it exactly;
// the classes are then converted to integers and combined with weights 1, 13, 169, 2197,
// 28561 in wrap-around 32-bit arithmetic (the exact result fits int32: |C| <= 2^14 K).
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
// 32 consecutive K values -> 16 bytes per digit plane.
__device__ __forceinline__ void pack32(const int8_t (&v)[32], const uint16_t* lut, uint4 (&out)[3]) {
  uint32_t w[3][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int d = 0; d < 3; ++d) w[d][q] = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t c = lut[(int)v[8 * q + u] + 128];
#pragma unroll
      for (int d = 0; d < 3; ++d) w[d][q] |= ((c >> (4 * d)) & 15u) << (4 * u);
    }
  }
#pragma unroll
  for (int d = 0; d < 3; ++d) out[d] = make_uint4(w[d][0], w[d][1], w[d][2], w[d][3]);
}

// axis 0: x rows x cols (K = cols); thread -> (row, 32-value chunk).
__global__ __launch_bounds__(256) void pack_rows_kernel(const int8_t* __restrict__ x,
                                                        int64_t rows, int64_t cols, int64_t ldx,
                                                        uint8_t* __restrict__ planes,
                                                        int64_t ldpb, int64_t plane_stride) {
  __shared__ uint16_t lut[256];
  lut[threadIdx.x] = d_limbs.codes[threadIdx.x];
  __syncthreads();
  const int64_t chunks = ldpb / 16;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= rows * chunks) return;
  const int64_t row = g / chunks;
  const int64_t h0 = (g - row * chunks) * 32;
  const int8_t* src = x + row * ldx;
  int8_t v[32];
#pragma unroll
  for (int u = 0; u < 32; ++u) v[u] = h0 + u < cols ? src[h0 + u] : (int8_t)0;
  uint4 out[3];
  pack32(v, lut, out);
#pragma unroll
  for (int d = 0; d < 3; ++d)
    *reinterpret_cast<uint4*>(planes + d * plane_stride + row * ldpb + h0 / 2) = out[d];
}

// axis 1: x rows x cols with K = rows; thread -> (column, 32-value chunk of K).
__global__ __launch_bounds__(256) void pack_cols_kernel(const int8_t* __restrict__ x,
                                                        int64_t rows, int64_t cols, int64_t ldx,
                                                        uint8_t* __restrict__ planes,
                                                        int64_t ldpb, int64_t plane_stride) {
  __shared__ uint16_t lut[256];
  lut[threadIdx.x] = d_limbs.codes[threadIdx.x];
  __syncthreads();
  const int64_t col = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  const int64_t h0 = ((int64_t)blockIdx.y * 4 + (threadIdx.x >> 6)) * 32;
  if (col >= cols || h0 >= 2 * ldpb) return;
  int8_t v[32];
#pragma unroll
  for (int u = 0; u < 32; ++u) v[u] = h0 + u < rows ? x[(h0 + u) * ldx + col] : (int8_t)0;
  uint4 out[3];
  pack32(v, lut, out);
#pragma unroll
  for (int d = 0; d < 3; ++d)
    *reinterpret_cast<uint4*>(planes + d * plane_stride + col * ldpb + h0 / 2) = out[d];
}

__device__ __forceinline__ v16f mfma_fp4(const v4i& a, const v4i& b, const v16f& c) {
  const v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  // cbsz = blgp = 4: both operands e2m1; scales 0x80 = 2^1 (E8M0) on both sides.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, 0x80, 0, 0x80);
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
// Workgroup tile 128 x 128, K step 64 (32 bytes per row per digit plane), 512 threads =
// 8 waves in 2 x 4, each wave 64 x 32 = 2 MFMA blocks x 5 weight classes (160 AGPRs).
// Digit planes of A and B go through registers into double-buffered LDS (2 x 24 KiB);
// LDS rows are 32 bytes with the two 16-byte halves swapped on rows with bit 3 set.
constexpr int FBM = 128, FBN = 128, FROW = 32;  // bytes per row per plane per K step
constexpr int kFThreads = 512;
constexpr int kPlaneA = FBM * FROW, kPlaneB = FBN * FROW;
constexpr int kStage = 3 * (kPlaneA + kPlaneB);  // 24 KiB

// 16 lanes read rows r..r+15 at the same half; rows 8 apart share banks without the XOR
// (gfx950 LDS: 64 four-byte banks, 16 lanes of 16 bytes per clock).
__device__ __forceinline__ int fswz(int row, int half) {
  return row * FROW + ((half ^ ((row >> 3) & 1)) << 4);
}

__global__ __launch_bounds__(kFThreads, 1) void fp4_gemm_kernel(
    int64_t m, int64_t n, int64_t ldpb, const uint8_t* __restrict__ pa, int64_t stride_a,
    const uint8_t* __restrict__ pb, int64_t stride_b, int32_t* __restrict__ c, int64_t ldc,
    int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - (blockIdx.x / tiles_n) * tiles_n;
  const int64_t row0 = (int64_t)tm * FBM, col0 = (int64_t)tn * FBN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 2;  // 0..1: rows wr*64
  const int wc = wave & 3;   // 0..3: cols wc*32

  // Global -> LDS assignment: 1536 chunks of 16 bytes (A planes, then B planes), 3 each.
  const uint8_t* gsrc[3];
  int ldst[3];
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int q = tid + kFThreads * s;
    const bool is_b = q >= 3 * FBM * 2;
    const int qq = is_b ? q - 3 * FBM * 2 : q;
    const int d = qq / (FBM * 2);  // FBM == FBN
    const int r = (qq >> 1) % FBM;
    const int h = qq & 1;
    int64_t gr = (is_b ? col0 : row0) + r;
    const int64_t last = (is_b ? n : m) - 1;
    gr = gr < last ? gr : last;
    gsrc[s] = (is_b ? pb + d * stride_b : pa + d * stride_a) + gr * ldpb + 16 * h;
    ldst[s] = (is_b ? 3 * kPlaneA + d * kPlaneB : d * kPlaneA) + fswz(r, h);
  }

  v16f acc[2][5];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int w = 0; w < 5; ++w)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][w][v] = 0.0f;

  v4i reg[3];
  const int64_t nk = ldpb / FROW;
  auto load_global = [&](int64_t t) {
#pragma unroll
    for (int s = 0; s < 3; ++s) reg[s] = *reinterpret_cast<const v4i*>(gsrc[s] + t * FROW);
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 3; ++s) *reinterpret_cast<v4i*>(lds + buf * kStage + ldst[s]) = reg[s];
  };
  const int frow = lane & 31, fhalf = lane >> 5;
  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int64_t t = 0; t < nk; ++t) {
    const int buf = (int)(t & 1);
    if (t + 1 < nk) load_global(t + 1);
    const uint8_t* base = lds + buf * kStage;
    v4i fa[2][3], fb[3];
#pragma unroll
    for (int d = 0; d < 3; ++d) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i][d] = *reinterpret_cast<const v4i*>(base + d * kPlaneA +
                                                 fswz(wr * 64 + i * 32 + frow, fhalf));
      fb[d] = *reinterpret_cast<const v4i*>(base + 3 * kPlaneA + d * kPlaneB +
                                            fswz(wc * 32 + frow, fhalf));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int da = 0; da < 3; ++da)
#pragma unroll
        for (int db = 0; db < 3; ++db)
          acc[i][da + db] = mfma_fp4(fa[i][da], fb[db], acc[i][da + db]);
    if (t + 1 < nk) store_lds(buf ^ 1);
    __syncthreads();
  }

  const int64_t col = col0 + wc * 32 + (lane & 31);
  if (col >= n) return;
  constexpr uint32_t kW[5] = {1u, 13u, 169u, 2197u, 28561u};
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = row0 + wr * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (row >= m) continue;
      uint32_t sum = 0;
#pragma unroll
      for (int w = 0; w < 5; ++w) sum += kW[w] * (uint32_t)(int32_t)acc[i][w][v];
      c[row * ldc + col] = (int32_t)sum;
    }
}

}  // namespace

int launch_fp4_pack(const int8_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                    uint8_t* planes, int64_t ldpb, int64_t plane_stride, hipStream_t s) {
  if (axis == 0) {
    if (rows <= 0) return OZK_OK;
    const int64_t threads = rows * (ldpb / 16);
    hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       x, rows, cols, ldx, planes, ldpb, plane_stride);
  } else {
    if (cols <= 0) return OZK_OK;
    dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((2 * ldpb / 32 + 3) / 4));
    hipLaunchKernelGGL(pack_cols_kernel, grid, dim3(256), 0, s, x, rows, cols, ldx, planes, ldpb,
                       plane_stride);
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
  const int64_t tiles_m = (m + FBM - 1) / FBM, tiles_n = (n + FBN - 1) / FBN;
  if (tiles_m * tiles_n > 0x7fffffff) return OZK_EUNSUPPORTED;
  hipLaunchKernelGGL(fp4_gemm_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kFThreads), 0, s,
                     m, n, ldpb, pa, stride_a, pb, stride_b, c, ldc, (int)tiles_n);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

}  // namespace ozk
