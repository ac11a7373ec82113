/*
 * ozk — Ozaki scheme II fp64 GEMM/GEMV emulation and exact INT8 products through FP4
 * limbs, for AMD Instinct MI355X (gfx950).  C ABI of libozk.so.
 *
 * Sources (cited by page title and part):
 *  [TME4] "The Missing Fourth Term for the Emulation Tensor Memory Equilibrium (TME)
 *         Model: The Residue Deconstruction Cost", arXiv 2610.10924v1, abstract.
 *         Ozaki scheme II emulates an fp64 matrix product with integer matrix
 *         products: every fp64 operand is scaled, rounded and reduced modulo each of r
 *         moduli (the deconstruction), one integer product runs per modulus (the
 *         tensor term), and a per-output reconstruction returns fp64.  GEMV and
 *         low-batch GEMV are memory bound; precomputed, stored residues move the
 *         deconstruction cost into HBM traffic.
 *  [AWE]  arXiv 2609.24519 listing (Nagoya University), English abstract.  Every
 *         product of the scheme is an exact integer product times a scale; 2 x FP4
 *         covers every residue mod 13, so an INT8 operand splits into three base-13
 *         digits (weights 1, 13, 169) stored as FP4, and INT8 x INT8 takes 9 FP4 GEMMs.
 *
 * Conventions for every entry point:
 *  - Matrices are row-major with a leading dimension (elements), as in PyTorch.
 *  - Pointers named A, B, C, X, Y, planes, exps, products, workspace are DEVICE
 *    pointers; pointers documented as "host" are host memory.  The caller owns all
 *    memory; the library never allocates device memory.  Scratch memory comes from a
 *    caller-provided workspace sized by the matching *_workspace_size query.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously; device faults surface at the caller's next synchronisation.
 *  - Arguments are validated before any HIP call; a failing check returns a negative
 *    status and enqueues nothing.  No C++ exception crosses the ABI.
 *  - Moduli: the first r of the pairwise-coprime integers <= 256 taken greedily from
 *    256 downwards (256, 255, 253, 251, 247, 241, 239, 233, 229, 227, 223, 217, 211,
 *    199, 197, 193, 191, 181, 179, 173); 1 <= r <= 20.
 *  - Scaling: a power of two per row of A and per column of B/X by the max rule
 *    e = P - 1 - ilogb(max |x|) (0 for an all-zero line), with bit budgets
 *    P_A = min(floor(beta/2), 76), P_B = min(beta - floor(beta/2), 76),
 *    beta = floor(log2((M-1)/2)) - ceil(log2 k), M the product of the moduli.  Scaled
 *    integers are rounded half to even and stay within 2^76 in magnitude.
 *  - Residues are symmetric: smod(x, m) in [-floor(m/2), ceil(m/2) - 1] (int8).
 *  - A line (row or column) holding Inf or NaN gets the exponent INT32_MIN, all-zero
 *    residues, and NaN in every output it touches.
 */
#ifndef OZK_H
#define OZK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OZK_OK 0
#define OZK_EINVAL (-1)       /* bad argument (null pointer, size, leading dimension, r) */
#define OZK_EWORKSPACE (-2)   /* workspace missing or smaller than the query returned */
#define OZK_ERANGE (-3)       /* k too large: int32 products or the bit budget would fail */
#define OZK_EHIP (-4)         /* a HIP launch failed */
#define OZK_EUNSUPPORTED (-5) /* valid request this build does not handle */
#define OZK_ENOSCRATCH (-6)   /* request needs more scratch than the allocation-free entry
                                 point's fixed array holds (OZK_NOALLOC_SCRATCH_BYTES) */

#define OZK_SCALING_MAX 0     /* scaling rule: per-line max (default of every entry point) */
#define OZK_SCALING_NORM 1    /* scaling rule: per-line 2-norm (Cauchy-Schwarz), *_ex only */

#define OZK_MAX_MODULI 20
#define OZK_MAX_K 131071      /* |residue product| <= 2^14: int32 sums stay exact */
#define OZK_PLANE_K 64        /* residue and limb planes pad K to a multiple of this */
#define OZK_NOALLOC_SCRATCH_BYTES (64ull << 20)  /* scratch of ozk_dgemv_noalloc, per GPU */

/* Library version (major * 10000 + minor * 100 + patch). */
int ozk_version(void);

/* Static description of a status code (never NULL). */
const char* ozk_status_string(int status);

/* Moduli of an r-modulus system: writes r int32 to `out` (host).  [TME4] abstract
 * ("each of the r moduli").  Returns OZK_EINVAL for r outside [1, 20] or out NULL. */
int ozk_moduli(int r, int32_t* out);

/* Bit budgets (P_A, P_B) of the scaling for r moduli and inner dimension k (host
 * outputs): the widths of the scaled, rounded integers of [TME4] abstract ("scaled,
 * rounded, and reduced modulo each of the r moduli"), chosen so that every dot product
 * of length k stays inside the range the r moduli determine exactly.  The pages fix no
 * rule; this is the max rule of the conventions above.  pa/pb may be NULL.  OZK_EINVAL
 * for r outside [1, 20] or k < 1; OZK_ERANGE when beta < 2 or k > OZK_MAX_K. */
int ozk_scaling_bits(int r, int64_t k, int32_t* pa, int32_t* pb);

/* Widths of either scaling rule (host outputs), the budget of the scaling step of
 * [TME4] abstract: OZK_SCALING_MAX gives (P_A, P_B) as above; OZK_SCALING_NORM gives
 * (alpha_A, alpha_B), the largest widths (alpha_A + alpha_B <= Q - 1, each <= 76) with
 * (2^aA + sqrt(k)/2)(2^aB + sqrt(k)/2) <= (M-1)/2, checked in exact integer arithmetic.
 * OZK_EINVAL for an unknown rule; otherwise the errors of ozk_scaling_bits. */
int ozk_scaling_bits_ex(int r, int64_t k, int scaling, int32_t* pa, int32_t* pb);

/* Leading dimension used for planes over an inner dimension k: round_up(k, 64). */
int64_t ozk_planes_ld(int64_t k);

/* ---------------------------------------------------------------- deconstruction
 * [TME4] abstract, the per-input deconstruction term: scale each line of x by a
 * power of two, round to an integer, reduce modulo each of the r moduli.
 *
 * axis 0 (A-side, per-row scaling with P_A):  x is rows x cols; K = cols.
 *     planes[l*plane_stride + i*ldp + h] = smod(RNE(x[i][h] 2^exps[i]), m_l)
 * axis 1 (B-side, per-column scaling with P_B): x is rows x cols with K = rows;
 *     planes[l*plane_stride + j*ldp + h] = smod(RNE(x[h][j] 2^exps[j]), m_l)
 *     (transposed, so K is contiguous as the products consume it).
 * In both cases entries with h in [K, ldp) are written as 0, exps has one int32 per
 * line (rows for axis 0, cols for axis 1), and the budget is that of inner dimension
 * k_budget (normally K).  ldp must be a multiple of 64 with ldp >= K; plane_stride >=
 * lines * ldp.  Reads x once for axis 0 when K <= 32768 (else twice); axis 1 reads x
 * twice (column maxima, then residues).
 */
int ozk_deconstruct_workspace_size(int64_t rows, int64_t cols, int axis, size_t* bytes);
int ozk_deconstruct(const double* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                    int r, int64_t k_budget, int8_t* planes, int64_t ldp,
                    int64_t plane_stride, int32_t* exps, void* workspace,
                    size_t workspace_bytes, void* stream);

/* The same with a choice of scaling rule (ozk_deconstruct is OZK_SCALING_MAX).
 * OZK_SCALING_NORM: exps[line] = alpha - 1 - (T + floor(u/2)) with alpha the width of
 * this operand (ozk_scaling_bits_ex), T = ilogb(max |x|) over the line, u = ilogb(RN(s
 * (1 + 2^-32))) and s = sum over the line of (x 2^-T)^2 in fp64, summed in a fixed
 * order (deterministic; the factor keeps RN(s (1 + 2^-32)) above the exact sum), so
 * that 2^e ||line||_2 < 2^alpha; 0 for an all-zero line, INT32_MIN for a line with
 * Inf/NaN.  The workspace of ozk_deconstruct_workspace_size covers both rules. */
int ozk_deconstruct_ex(const double* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                       int r, int64_t k_budget, int scaling, int8_t* planes, int64_t ldp,
                       int64_t plane_stride, int32_t* exps, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- modular products
 * [TME4] abstract, the tensor term; [AWE] abstract, each product is an error-free
 * integer matrix product.  For l < r:
 *     products[l*stride_p + i*ldp_out + j] = sum_{h < kp} pa[l*stride_a + i*kp + h]
 *                                                       * pb[l*stride_b + j*kp + h]
 * exactly in int32 (int8 planes as written by ozk_deconstruct; kp a multiple of 64,
 * kp <= OZK_MAX_K rounded up, i.e. at most 131072).  Exact while every sum fits int32,
 * which planes from ozk_deconstruct (at most 131071 live K positions, the padding zero)
 * always do; caller-made planes with kp = 131072 must keep one K position zero in A or
 * B, or a line of 131072 terms (-128)(-128) = 2^31 wraps.  m x n outputs per modulus;
 * ldp_out >= n. */
int ozk_modular_products(int64_t m, int64_t n, int64_t kp, int r, const int8_t* pa,
                         int64_t stride_a, const int8_t* pb, int64_t stride_b,
                         int32_t* products, int64_t ldp_out, int64_t stride_p, void* stream);

/* Same products reduced to their symmetric residues modulo m_l, as int8 (what the
 * reconstruction consumes; the kernel ozk_dgemm runs):
 *     residues[l*stride_r + i*ldr + j] = smod(sum_h pa[..] * pb[..], m_l)          */
int ozk_modular_residues(int64_t m, int64_t n, int64_t kp, int r, const int8_t* pa,
                         int64_t stride_a, const int8_t* pb, int64_t stride_b,
                         int8_t* residues, int64_t ldr, int64_t stride_r, void* stream);

/* ---------------------------------------------------------------- reconstruction
 * [TME4] abstract, the per-output reconstruction term.  For each output, the r
 * int32 products are reduced modulo their moduli, lifted exactly by the Chinese
 * Remainder Theorem to the integer X with |X| <= 2^Q (Q = floor(log2((M-1)/2)), the
 * range the bit budget keeps every emulated dot product in), and
 *     C[i][j] = RN(X * 2^-(exps_a[i] + exps_b[j]))
 * rounded once to nearest even (subnormal results included; overflow gives +-Inf).
 * Residues of an integer outside that range give an unspecified finite value.
 * A NONFINITE (INT32_MIN) exponent gives NaN.  ldp_in >= n, ldc >= n. */
int ozk_reconstruct(int64_t m, int64_t n, int r, const int32_t* products, int64_t ldp_in,
                    int64_t stride_p, const int32_t* exps_a, const int32_t* exps_b,
                    double* C, int64_t ldc, void* stream);

/* ---------------------------------------------------------------- emulated DGEMM
 * [TME4] abstract (Ozaki scheme II: deconstruction, one integer product per modulus,
 * per-output reconstruction); [AWE] abstract (each product an error-free integer matrix
 * product times a scale factor).
 * C = A B (m x n, A m x k, B k x n, no alpha/beta) through r moduli: deconstruction
 * of A (rows) and B (columns), r int8 MFMA products with the residue epilogue, CRT
 * reconstruction.  The result equals RN(2^-(e_i+f_j) sum_h a'_ih b'_hj) with the
 * sum exact.  m, n >= 0; 1 <= k <= OZK_MAX_K; lda >= k, ldb >= n, ldc >= n.  The
 * workspace (device, 256-byte aligned, at least ozk_dgemm_workspace_size bytes) holds
 * the residue planes of A and B, the product residues and the exponents; its contents
 * are scratch on return.  OZK_EWORKSPACE when it is missing or short; nothing is
 * enqueued on any error. */
int ozk_dgemm_workspace_size(int64_t m, int64_t n, int64_t k, int r, size_t* bytes);
int ozk_dgemm(int64_t m, int64_t n, int64_t k, const double* A, int64_t lda,
              const double* B, int64_t ldb, double* C, int64_t ldc, int r,
              void* workspace, size_t workspace_bytes, void* stream);

/* The same with a choice of scaling rule (ozk_dgemm is OZK_SCALING_MAX); the workspace
 * of ozk_dgemm_workspace_size covers both.  OZK_SCALING_NORM scales rows of A and
 * columns of B by their 2-norms (see ozk_deconstruct_ex), which keeps more bits of
 * lines whose entries differ widely in magnitude for the same r. */
int ozk_dgemm_ex(int64_t m, int64_t n, int64_t k, const double* A, int64_t lda,
                 const double* B, int64_t ldb, double* C, int64_t ldc, int r, int scaling,
                 void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- emulated DGEMV
 * Y = A X for A m x k and X k x nrhs (1 <= nrhs <= 32): the memory-bound GEMV and
 * low-batch GEMV of [TME4] abstract.  Same arithmetic and result as ozk_dgemm.
 * mode 0 (on the fly): A is streamed as fp64 and deconstructed in registers; A_exps
 *        may be NULL (row exponents are then computed first, one extra pass over A)
 *        or hold exponents from ozk_deconstruct(axis 0, k_budget = k).
 * mode 1 (stored):     A_planes/A_exps come from ozk_deconstruct(A, axis 0,
 *        k_budget = k) with leading dimension ldp and plane stride plane_stride; A
 *        may be NULL.  r bytes per element of A are streamed.  [TME4] abstract: the
 *        stored residues move the deconstruction cost into the bandwidth term. */
int ozk_dgemv_workspace_size(int64_t m, int64_t k, int64_t nrhs, int r, int mode,
                             size_t* bytes);
int ozk_dgemv(int64_t m, int64_t k, int64_t nrhs, const double* A, int64_t lda,
              const int8_t* A_planes, int64_t ldp, int64_t plane_stride,
              const int32_t* A_exps, const double* X, int64_t ldx, double* Y, int64_t ldy,
              int r, int mode, void* workspace, size_t workspace_bytes, void* stream);

/* ozk_dgemv_noalloc: for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  ozk_dgemv with
 * the same arguments, result and errors, except that there is no workspace: the
 * scratch lives in a fixed device array of the library, OZK_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU, held by each GPU the library runs on until the process ends.  A
 * request whose ozk_dgemv_workspace_size exceeds it returns OZK_ENOSCRATCH (nothing is
 * enqueued); 64 MiB covers the 32768 x 32768 GEMV at r = 14 with 1, 8 or 32 columns in
 * both modes.  The call uses the scratch of the current device, so `stream` must belong
 * to the current device.  It allocates nothing and calls no allocating routine.  Every
 * call on one GPU shares that GPU's array: calls ordered on one stream are safe, calls
 * that may overlap in time on one GPU (other streams, other threads) race. */
int ozk_dgemv_noalloc(int64_t m, int64_t k, int64_t nrhs, const double* A, int64_t lda,
                      const int8_t* A_planes, int64_t ldp, int64_t plane_stride,
                      const int32_t* A_exps, const double* X, int64_t ldx, double* Y,
                      int64_t ldy, int r, int mode, void* stream);

/* ---------------------------------------------------------------- emulated SpMV
 * y = A x for A rows x cols in CSR (row_ptr: rows + 1 int32 offsets into col_idx and
 * vals, nnz entries; column indices need not be sorted), x of cols entries, through r
 * moduli: the sparse matrix-vector product [TME4] abstract lists among the memory-bound
 * kernels of emulation.  Rows of A are scaled by the max rule over their nonzeros with
 * the budget of dot products of max_row_nnz terms (ozk_scaling_bits(r, max_row_nnz)),
 * x by one exponent; exact int32 row sums per modulus; CRT lift and one rounding, as
 * ozk_dgemm.  An empty row gives +0.  A row whose row_ptr extent is not inside
 * [0, nnz], that has more than max_row_nnz entries, holds a column index outside
 * [0, cols) or holds Inf/NaN gives NaN (nothing is read through a bad index); Inf/NaN
 * in x makes every y NaN.  All pointers are device pointers; 1 <= max_row_nnz <=
 * OZK_MAX_K; nnz, rows and cols below 2^31. */
int ozk_spmv_csr_workspace_size(int64_t rows, int64_t cols, int r, size_t* bytes);
int ozk_spmv_csr(int64_t rows, int64_t cols, int64_t nnz, const int32_t* row_ptr,
                 const int32_t* col_idx, const double* vals, int64_t max_row_nnz,
                 const double* x, double* y, int r, void* workspace, size_t workspace_bytes,
                 void* stream);

/* ---------------------------------------------------------------- FP4-limb INT8 GEMM
 * [AWE] abstract: x = d0 + 13 d1 + 169 d2 with every digit in
 * S = {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12}; the digit of residue rho (mod 13) is
 * the element of S of least magnitude congruent to rho; digit d is stored as the
 * e2m1 code of d/2, two codes per byte, the even K index in the low nibble.
 *
 * ozk_fp4limb_pack:  axis 0: x rows x cols (K = cols) ->
 *        planes[d*plane_stride + i*ldp_bytes + h/2], nibble h&1, for digit d in 0..2;
 *   axis 1: x rows x cols (K = rows) -> planes[d*plane_stride + j*ldp_bytes + h/2].
 *   Codes for h in [K, 2*ldp_bytes) are 0.  ldp_bytes multiple of 32, >= round_up(K,64)/2.
 * ozk_fp4limb_products: the 9 digit products, exact:
 *   products[(3*da+db)*stride_p + i*ldp_out + j] = sum_h D_da(A)[i][h] D_db(B)[h][j]
 *   from packed planes with K extent kp = 2*ldp_bytes (a multiple of 64).
 * ozk_int8gemm_fp4limb: C = A B exactly in int32 (A m x k, B k x n int8), as the sum
 *   of the 9 FP4 products weighted by 13^(da+db).  k <= OZK_MAX_K. */
int ozk_fp4limb_pack(const int8_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                     uint8_t* planes, int64_t ldp_bytes, int64_t plane_stride, void* stream);
int ozk_fp4limb_products(int64_t m, int64_t n, int64_t ldp_bytes, const uint8_t* planes_a,
                         int64_t stride_a, const uint8_t* planes_b, int64_t stride_b,
                         int32_t* products, int64_t ldp_out, int64_t stride_p, void* stream);
int ozk_int8gemm_fp4limb_workspace_size(int64_t m, int64_t n, int64_t k, size_t* bytes);
int ozk_int8gemm_fp4limb(int64_t m, int64_t n, int64_t k, const int8_t* A, int64_t lda,
                         const int8_t* B, int64_t ldb, int32_t* C, int64_t ldc,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- 6-product FP4 INT8 GEMM
 * [AWE] abstract: with free integer limb weights and stored planes that combine limbs, an
 * INT8 x INT8 product takes 6 FP4 matrix products instead of 9.  Encoding used here: x =
 * a0 + 29 a1 + 37 a2 with the limbs a_i and their pairwise sums a0+a1, a0+a2, a1+a2 all in
 * S (each at most 6 in magnitude); of the triples that encode x, the one whose six plane
 * values have the smallest largest magnitude, then sum of squares, then (a0, a1, a2)
 * lexicographically.  C = A B = sum_t coef_t P_t over the 6 plane products, coef = (-65,
 * -261, 259, 29, 37, 1073) (the three-term Karatsuba identity).
 *
 * Packed layout: one line per row of A (axis 0, K = cols) or column of B (axis 1, K =
 * rows); K in steps of 64 codes, step s of a line at bytes 192 s .. 192 s + 191, plane t
 * (a0, a1, a2, a0+a1, a0+a2, a1+a2) at byte 32 t of the step, value d stored as the e2m1
 * code of d/2, two codes per byte with the even K index in the low nibble; codes past K
 * are 0.  ozk_fp4awe_line_bytes(k) = 192 ceil(k / 64) is the smallest line stride.
 *
 * ozk_fp4awe_pack: planes[line * ld_line + ...] (device, 16-byte aligned), ld_line >=
 *   ozk_fp4awe_line_bytes(K) and a multiple of 16; K <= OZK_MAX_K.
 * ozk_fp4awe_products: the 6 exact plane products, products[t*stride_p + i*ldp_out + j] =
 *   sum_h U_t(A)[i][h] V_t(B)[h][j] (int32), from packed lines of A (m lines, stride lda)
 *   and B (n lines, stride ldb) over inner dimension k <= OZK_MAX_K.
 * ozk_int8gemm_fp4awe: C = A B exactly in int32 (A m x k, B k x n int8 row-major), packing
 *   both operands into the workspace (ozk_int8gemm_fp4awe_workspace_size bytes, 256-byte
 *   aligned) and summing the 6 weighted plane products.  k <= OZK_MAX_K (fp32 partial
 *   sums stay exact: each elementary product is at most 36). */
int64_t ozk_fp4awe_line_bytes(int64_t k);
int ozk_fp4awe_pack(const int8_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                    uint8_t* planes, int64_t ld_line, void* stream);
int ozk_fp4awe_products(int64_t m, int64_t n, int64_t k, const uint8_t* planes_a, int64_t lda,
                        const uint8_t* planes_b, int64_t ldb, int32_t* products,
                        int64_t ldp_out, int64_t stride_p, void* stream);
int ozk_int8gemm_fp4awe_workspace_size(int64_t m, int64_t n, int64_t k, size_t* bytes);
int ozk_int8gemm_fp4awe(int64_t m, int64_t n, int64_t k, const int8_t* A, int64_t lda,
                        const int8_t* B, int64_t ldb, int32_t* C, int64_t ldc, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- 4-product FP4 INT4 x INT8 GEMM
 * [AWE] abstract: with free integer limb weights and stored planes that combine limbs, an
 * INT4 x INT8 product takes 4 FP4 matrix products.  Encoding used here: an int4 x = a0 +
 * 5 a1 and an int8 y = b0 + 5 b1 + 25 b2 are the values at (5, 1) of the forms X(p, q) =
 * q a0 + p a1 and Y(p, q) = q^2 b0 + p q b1 + p^2 b2; the stored planes are X and Y at the
 * points (0, 1), (1, 0), (1, 1), (1, 2): U = (a0, a1, a0+a1, 2 a0+a1) for the int4 operand,
 * V = (b0, b2, b0+b1+b2, 4 b0+2 b1+b2) for the int8 operand, all in S (U at most 4 and V
 * at most 12 in magnitude); of the limb tuples that encode a value, the one whose planes
 * have the smallest largest magnitude, then sum of squares, then the smallest limbs
 * lexicographically.  C = A B = 36 P_0 + 90 P_1 + 45 P_2 - 10 P_3 over the plane products
 * P_t = U_t(A) V_t(B) (interpolation of the cubic form X Y at the four points).  An int4
 * value is the low four bits of its byte, two's complement: an int8 array of values in
 * [-8, 7] is read as it is, any other byte by its low nibble.
 *
 * Packed layout: one line per row (axis 0, K = cols) or column (axis 1, K = rows) of x; K
 * in steps of 64 codes, step s of a line at bytes 128 s .. 128 s + 127, plane t at byte
 * 32 t of the step, value d stored as the e2m1 code of d/2, two codes per byte with the
 * even K index in the low nibble; codes past K are 0.  ozk_fp4awe4_line_bytes(k) = 128
 * ceil(k / 64) is the smallest line stride.
 *
 * ozk_fp4awe4_pack: the U planes of an int4 matrix (int4 = 1) or the V planes of an int8
 *   matrix (int4 = 0); planes[line * ld_line + ...] (device, 16-byte aligned), ld_line >=
 *   ozk_fp4awe4_line_bytes(K) and a multiple of 16; K <= OZK_MAX_K.
 * ozk_fp4awe4_products: the 4 exact plane products, products[t*stride_p + i*ldp_out + j] =
 *   sum_h U_t(A)[i][h] V_t(B)[h][j] (int32), from packed lines of A (m lines, stride lda)
 *   and B (n lines, stride ldb) over inner dimension k <= OZK_MAX_K.
 * ozk_int4int8gemm_fp4awe: C = A B exactly in int32 (A m x k int4 values one per byte, B
 *   k x n int8, both row-major), packing both operands into the workspace
 *   (ozk_int4int8gemm_fp4awe_workspace_size bytes, 256-byte aligned) and summing the 4
 *   weighted plane products (products 1 and 2, whose weights are 90 and 45, summed in one
 *   fp32 accumulator).  k <= OZK_MAX_K (fp32 partial sums stay exact: per K value the
 *   plane products are at most 48 in magnitude, and 2 P1 + P2 at most 27). */
int64_t ozk_fp4awe4_line_bytes(int64_t k);
int ozk_fp4awe4_pack(const int8_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis,
                     int int4, uint8_t* planes, int64_t ld_line, void* stream);
int ozk_fp4awe4_products(int64_t m, int64_t n, int64_t k, const uint8_t* planes_a,
                         int64_t lda, const uint8_t* planes_b, int64_t ldb, int32_t* products,
                         int64_t ldp_out, int64_t stride_p, void* stream);
int ozk_int4int8gemm_fp4awe_workspace_size(int64_t m, int64_t n, int64_t k, size_t* bytes);
int ozk_int4int8gemm_fp4awe(int64_t m, int64_t n, int64_t k, const int8_t* A, int64_t lda,
                            const int8_t* B, int64_t ldb, int32_t* C, int64_t ldc,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- measurement support
 * ozk_dgemm_ex_timed: ozk_dgemm_ex that also has the launch of the r residue products
 *   record its start and end in the caller's two hipEvent_t handles (gemm_start,
 *   gemm_stop: both NULL or both events created with timing on the stream's device; the
 *   launch records them itself, hipExtLaunchKernel, so no extra stream commands are
 *   added), so that a benchmark can time that kernel inside the steps it times.  Same
 *   arguments, result and errors as ozk_dgemm_ex; one of the two events NULL without the
 *   other: OZK_EINVAL.  The events stay owned by the caller. */
int ozk_dgemm_ex_timed(int64_t m, int64_t n, int64_t k, const double* A, int64_t lda,
                       const double* B, int64_t ldb, double* C, int64_t ldc, int r, int scaling,
                       void* workspace, size_t workspace_bytes, void* stream,
                       void* gemm_start, void* gemm_stop);

#ifdef __cplusplus
}
#endif

#endif /* OZK_H */
