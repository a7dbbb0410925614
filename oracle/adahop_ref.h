/*
 * AdaHOP oracle: a plain, slow CPU implementation of the per-GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this library; only the tests, the smoke check and the benchmark's CPU
 * baseline use it. It shares no code, header, table or constant with the GPU
 * library.
 *
 * Source: "AdaHOP: Fast and Accurate Low-Precision Training via
 * Outlier-Pattern-Aware Rotation" (arXiv 2604.02525): abstract; Fig. 2; Fig. 5;
 * Table 1; Fig. 9 and the appendix list of its four kernels (FOID; IHT and
 * quantization; fused MXFP4+BF16 GEMM; fused scatter-add). MXFP4 follows the
 * OCP Microscaling Formats (MX) v1.0 specification, which is what the name
 * denotes: E2M1 elements, one E8M0 scale per 32 elements.
 *
 * Conventions (identical on purpose to the GPU library's public contract, so
 * that results can be compared; the two are written separately):
 *   - bf16 tensors are uint16 bit patterns, row-major, leading dim `ld`.
 *   - Textbook frame of a GEMM: C[m,n] = A[m,K] * B[K,n].
 *   - Packed MXFP4 operand: codes [outer][K/2] (element 2j in the low nibble),
 *     scales [outer][K/32] (E8M0 bytes); K, the contraction dim, contiguous.
 *     For A, outer = m; for B, outer = n.
 * All functions return 0 on success and a negative value on bad arguments.
 */
#ifndef ADAHOP_REF_H
#define ADAHOP_REF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { REF_PAT_NONE = 0, REF_PAT_ROW = 1, REF_PAT_COL = 2 };
enum { REF_OP_FWD = 0, REF_OP_DGRAD = 1, REF_OP_WGRAD = 2 };
enum { REF_ROUTE_BF16 = 0, REF_ROUTE_IHT = 1, REF_ROUTE_OE_LEFT = 2, REF_ROUTE_OE_RIGHT = 3,
       REF_ROUTE_OE_INNER = 4, REF_ROUTE_MXFP4 = 5 };
enum { REF_AXIS_ROWS = 0, REF_AXIS_COLS = 1 };

/* Route of one GEMM from its storage-frame operand patterns. */
int adahop_ref_route(int op, int pat_lhs, int pat_rhs);
/* For an OE route: which stored operand FOID scans (0 = lhs, 1 = rhs) and
 * whether its candidate lines are rows or columns. */
int adahop_ref_scan_target(int op, int route, int* tensor, int* axis);

/* FOID. Candidate lines are rows (axis ROWS) or columns (axis COLS) of t.
 * var_out (optional, one per candidate) receives each line's probe variance. */
int adahop_ref_foid(const uint16_t* t, int64_t rows, int64_t cols, int64_t ld, int axis,
                    int probe, int k, int32_t* idx_out, double* var_out);

/* 32-point fast Walsh-Hadamard transform of one block in fp32, orthonormal. */
void adahop_ref_fwht32(float y[32]);

/* E2M1 magnitude code (0..7) of a non-negative, already scaled value. */
int adahop_ref_e2m1_magnitude(double v);
/* Signed value of a 4-bit E2M1 code, without the block scale. */
double adahop_ref_e2m1_value(int code);
/* One 32-element block: E8M0 scale byte and 16 bytes of packed codes. */
void adahop_ref_mx_block(const float y[32], uint8_t codes[16], uint8_t* scale);

/* Zero lines, optional IHT (hadamard_block 32, or 0 for none), MXFP4 quantize.
 * contract COLS: blocks run along rows (K = cols, outer = rows);
 * contract ROWS: blocks run down columns (K = rows, outer = cols).
 * zero_axis: zero_idx names rows (ROWS) or columns (COLS) of src.
 * gathered (optional): the zeroed lines in bf16, one line per row:
 * [nzero][cols] for rows, [nzero][rows] for columns. */
int adahop_ref_iht_quant(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld,
                         int contract, int hadamard_block, const int32_t* zero_idx,
                         int32_t nzero, int zero_axis, uint8_t* codes, uint8_t* scales,
                         uint16_t* gathered);

/* fp64 product of two packed MXFP4 operands on selected outputs:
 * C[a][b] for i = rows[a], j = cols[b]; absC (optional) = sum of |products|. */
int adahop_ref_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales,
                       const uint8_t* b_codes, const uint8_t* b_scales, int64_t K,
                       const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                       double* C, double* absC);

/* fp64 product of two bf16 operands in the textbook frame on selected outputs.
 * A(i,t) = a[i*lda + t] (a_trans 0) or a[t*lda + i] (a_trans 1);
 * B(t,j) = b[t*ldb + j] (b_trans 0) or b[j*ldb + t] (b_trans 1). */
int adahop_ref_gemm_bf16(const uint16_t* a, int64_t lda, int a_trans,
                         const uint16_t* b, int64_t ldb, int b_trans, int64_t K,
                         const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                         double* C, double* absC);

/* Running-error terms of an fp32 accumulation of the same products, on
 * selected outputs (a test tolerance, not part of the method): with S_j the
 * exact sum of the first j*step products in contraction order and
 * R_j = max_{i<=j} |S_i|, walk = sum_j (|S_j| + R_j) and rmax = the last R_j.
 * u * walk bounds, to first order, the rounding error of an fp32 accumulator
 * that adds `step` products (or fewer) at a time in contraction order, also
 * when the contraction is cut into contiguous parts added afterwards. */
int adahop_ref_walk_mx(const uint8_t* a_codes, const uint8_t* a_scales,
                       const uint8_t* b_codes, const uint8_t* b_scales, int64_t K, int64_t step,
                       const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                       double* walk, double* rmax);
int adahop_ref_walk_bf16(const uint16_t* a, int64_t lda, int a_trans,
                         const uint16_t* b, int64_t ldb, int b_trans, int64_t K, int64_t step,
                         const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                         double* walk, double* rmax);

/* Dequantize a packed operand to fp64 [outer][K]. */
int adahop_ref_dequant(const uint8_t* codes, const uint8_t* scales, int64_t outer, int64_t K,
                       double* out);

/* Threads the OpenMP loops may use (1 if built without OpenMP). */
int adahop_ref_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif
