// Internal declarations of the ozk library: constant tables, launch helpers and the
// per-element arithmetic shared by the kernels.  Nothing here is part of the C ABI.
//
// Method: Ozaki scheme II emulation of fp64 matrix products, as summarised in "The
// Missing Fourth Term for the Emulation Tensor Memory Equilibrium (TME) Model: The
// Residue Deconstruction Cost" (arXiv 2610.10924), abstract: operands are scaled,
// rounded and reduced modulo r moduli; one integer matrix product per modulus; a
// per-output reconstruction returns fp64.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ozk.h"

namespace ozk {

constexpr int kMaxModuli = 20;
constexpr int kPlaneK = 64;          // residue planes: K padded to a multiple of this
constexpr int kExpNonfinite = INT32_MIN;
constexpr int kMaxLimbs = 4;         // CRT limbs of 2^40
constexpr double kMagic = 6755399441055744.0;  // 1.5 * 2^52: x + kMagic rounds x to an integer

// Per-modulus constants for the residue kernels (passed by value as kernel arguments).
struct ResidueConsts {
  int r;
  int wide;                     // 1 when scaled integers may exceed 2^51 (split path)
  double m[kMaxModuli];         // moduli as doubles
  double inv[kMaxModuli];       // RN(1/m)
  double c32[kMaxModuli];       // smod(2^32, m)
};

// Constants of the CRT reconstruction.
struct CrtConsts {
  int r;
  int limbs;                          // 3 or 4 limbs of 2^40
  int32_t mod[kMaxModuli];            // moduli
  double inv[kMaxModuli];             // RN(1/m)
  double frac[kMaxModuli];            // RN(E_l / M) = RN(w_l / m_l)
  double e_limb[kMaxModuli][kMaxLimbs];  // E_l in base 2^40, least significant first
  double m_limb[kMaxLimbs];           // M in base 2^40
};

// Host side (rns_host.cpp)
// Largest width of a scaled integer under either rule: |a'| <= 2^76 keeps the wide residue
// arithmetic exact (|hi smod(2^32, m) + lo| <= 2^44 * 127 + 2^32 < 2^51).
constexpr int kWidthCap = 76;
int moduli_list(int r, int32_t* out);
int scaling_bits(int r, int64_t k, int* pa, int* pb);
// Norm rule widths (alpha_A, alpha_B): (2^aA + sqrt(k)/2)(2^aB + sqrt(k)/2) <= (M-1)/2.
int scaling_bits_norm(int r, int64_t k, int* pa, int* pb);
// Widths of either rule (OZK_SCALING_MAX: P_A, P_B; OZK_SCALING_NORM: alpha_A, alpha_B).
int scaling_widths(int scaling, int r, int64_t k, int* wa, int* wb);
// Either rule bounds every scaled integer by 2^width (max rule: |x| 2^e < 2^P; norm rule:
// |x| 2^e <= ||x||_2 2^e < 2^alpha; round-to-nearest reaches at most the power of two),
// so `width` alone picks the narrow or wide residue arithmetic.
const ResidueConsts* residue_consts(int r, int p_bits);
const CrtConsts* crt_consts(int r);

inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Every argument check of ozk_dgemv except the workspace's (no HIP call): OZK_OK or the
// status ozk_dgemv would return.
int dgemv_validate(int64_t m, int64_t k, int64_t nrhs, const double* A, int64_t lda,
                   const int8_t* A_planes, int64_t ldp, int64_t plane_stride,
                   const int32_t* A_exps, const double* X, int64_t ldx, const double* Y,
                   int64_t ldy, int r, int mode);
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Launchers (each defined next to its kernels).  All return OZK_OK or OZK_EHIP.
int launch_fill_u64(uint64_t* p, int64_t n, uint64_t v, hipStream_t s);
int launch_absmax(const double* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                  uint64_t* maxbits, hipStream_t s);
// given_exps: exps already holds the exponents (norm rule, width = alpha); else the max
// rule with width = P from maxbits, written to exps.
int launch_residues(const double* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                    int r, int width, const uint64_t* maxbits, int8_t* planes, int64_t ldp,
                    int64_t plane_stride, int32_t* exps, int given_exps, hipStream_t s);
int launch_residues_rows_fused(const double* x, int64_t rows, int64_t cols, int64_t ldx,
                               int r, int scaling, int width, int8_t* planes, int64_t ldp,
                               int64_t plane_stride, int32_t* exps, hipStream_t s);
bool rows_fused_supported(int64_t cols);
// A (rows, fused) and B (column residues) of one product in a single launch, for k <=
// 8192 and equal residue arithmetic on both sides; B's exponents (norm rule) or maxima
// (max rule, maxbits_b) must already be in place.  OZK_EUNSUPPORTED when not
// applicable (the caller then deconstructs the operands one after the other).
int launch_deconstruct_pair(const double* a, int64_t m, int64_t k, int64_t lda, const double* b,
                            int64_t n, int64_t ldb, int r, int scaling, int width_a, int width_b,
                            const uint64_t* maxbits_b, int8_t* planes_a, int8_t* planes_b,
                            int64_t kp, int32_t* exps_a, int32_t* exps_b, hipStream_t s);
// Norm rule, unfused paths: per-chunk maxima and scaled sums of squares into pmax/ps
// (norm_chunks(...) entries per line each), then the exponents from them.
int64_t norm_chunks(int64_t rows, int64_t cols, int axis);
int launch_norm_exps(const double* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                     int alpha, uint64_t* pmax, double* ps, int32_t* exps, hipStream_t s);
// Emulated SpMV: x's exponent (chunk maxima in x_partial, ceil(cols / 2048) entries) and
// residues xres[cols][16 or 32] (r <= 16 or not), then one thread per CSR row: row
// exponents (max rule, width p_a) and the symmetric residues of the row sums, written as
// res[l * rows + i]; rows with a bad extent, more than kmax entries or a column index
// outside [0, cols) get the exponent INT32_MIN.
int launch_spmv(int64_t rows, int64_t cols, int64_t nnz, const int32_t* row_ptr,
                const int32_t* col_idx, const double* vals, int64_t kmax, const double* x,
                int r, int p_a, int p_b, uint64_t* x_partial, int32_t* x_exp, int8_t* xres,
                int8_t* res, int32_t* exps, hipStream_t s);
// Row (axis 0) or column (axis 1) exponents only, through maxbits scratch.
int launch_line_exps(const double* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                     int p_bits, uint64_t* maxbits, int32_t* exps, hipStream_t s);

int launch_gemv_stored(int64_t m, int64_t kp, int r, const int8_t* ap, int64_t lda_p,
                       int64_t a_stride, const int8_t* xp, int64_t x_stride, int nrhs,
                       int8_t* res, hipStream_t s);
int launch_gemv_fly(const double* a, int64_t m, int64_t k, int64_t lda, const int32_t* exps,
                    int r, int p_bits, const int8_t* xp, int64_t ldp, int64_t x_stride, int nrhs,
                    int8_t* res, hipStream_t s);

// On-the-fly GEMV through base-256 digits of the scaled integers (scaling bits <= 50,
// at most 256 output columns r * nrhs).
bool gemv_digits_supported(int p_bits, int64_t ncols);
size_t gemv_digits_workspace(int64_t m, int64_t kp, int r, int64_t nrhs, size_t* xd_bytes,
                             size_t* corr_bytes, size_t* part_bytes);
int launch_gemv_digits(const double* a, int64_t m, int64_t k, int64_t lda, const int32_t* exps,
                       int r, const int8_t* xp, int64_t kp, int64_t x_stride, int nrhs,
                       int8_t* xd, int32_t* psum, int8_t* part, int8_t* res, hipStream_t s);

int launch_fp4_pack(const int8_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                    uint8_t* planes, int64_t ldpb, int64_t plane_stride, hipStream_t s);
int launch_fp4_products(int64_t m, int64_t n, int64_t ldpb, const uint8_t* pa, int64_t stride_a,
                        const uint8_t* pb, int64_t stride_b, int32_t* out, int64_t ldo,
                        int64_t stride_o, hipStream_t s);
int launch_fp4_gemm(int64_t m, int64_t n, int64_t ldpb, const uint8_t* pa, int64_t stride_a,
                    const uint8_t* pb, int64_t stride_b, int32_t* c, int64_t ldc, hipStream_t s);

// The 6-product FP4 engine (fp4awe.hip): bytes of one packed line over inner dimension k
// (192 per K step of 64 codes), packer (axis 0: lines are rows of x, K = cols; axis 1:
// lines are columns, K = rows), the 6 plane products (test path) and the fused GEMM.
int64_t awe_line_bytes(int64_t k);
int launch_awe_pack(const int8_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                    uint8_t* out, int64_t ld_line, hipStream_t s);
int launch_awe_products(int64_t m, int64_t n, int64_t steps, const uint8_t* pa, int64_t lda,
                        const uint8_t* pb, int64_t ldb, int32_t* out, int64_t ldo,
                        int64_t stride_o, hipStream_t s);
int launch_awe_gemm(int64_t m, int64_t n, int64_t steps, const uint8_t* pa, int64_t lda,
                    const uint8_t* pb, int64_t ldb, int32_t* c, int64_t ldc, hipStream_t s);
// The 4-product INT4 x INT8 FP4 engine (fp4awe4.hip): bytes of one packed line over inner
// dimension k, packers (int4: A-side planes of the low nibbles, else B-side planes of int8
// values), plane products, fused GEMM.
int64_t awe4_line_bytes(int64_t k);
int launch_awe4_pack(const int8_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                     int int4, uint8_t* out, int64_t ld_line, hipStream_t s);
int launch_awe4_products(int64_t m, int64_t n, int64_t steps, const uint8_t* pa, int64_t lda,
                         const uint8_t* pb, int64_t ldb, int32_t* out, int64_t ldo,
                         int64_t stride_o, hipStream_t s);
int launch_awe4_gemm(int64_t m, int64_t n, int64_t steps, const uint8_t* pa, int64_t lda,
                     const uint8_t* pb, int64_t ldb, int32_t* c, int64_t ldc, hipStream_t s);

enum GemmEpilogue { kEpiProducts = 0, kEpiResidues = 1 };
// ev_start / ev_stop (optional, both or neither): caller events the launch records its
// start and end in (hipExtLaunchKernel), for timing the products inside a step.
int launch_gemm_i8(int64_t m, int64_t n, int64_t kp, int r, const int8_t* pa, int64_t stride_a,
                   const int8_t* pb, int64_t stride_b, void* out, int64_t ldo, int64_t stride_o,
                   int epilogue, hipStream_t s, hipEvent_t ev_start = nullptr,
                   hipEvent_t ev_stop = nullptr);

int launch_crt(int64_t m, int64_t n, int r, const void* res, int res_is_i32, int64_t ldr,
               int64_t stride_r, const int32_t* ea, const int32_t* eb, double* c, int64_t ldc,
               hipStream_t s);

}  // namespace ozk
