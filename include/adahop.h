/*
 * adahop.h -- C ABI of the AdaHOP per-GEMM hot path on MI355X (gfx950).
 *
 * The method is the one of "AdaHOP: Fast and Accurate Low-Precision Training
 * via Outlier-Pattern-Aware Rotation" (arXiv 2604.02525). Its Fig. 9 and the
 * appendix list of its kernels give four stages per GEMM:
 *   1. FOID: the outlier lines of one operand, chosen by the variance of their
 *      first 64 elements (adahop_detect);
 *   2. IHT and quantization: zero those lines, rotate the residual by a
 *      32-point Hadamard transform along the inner dimension, quantize to
 *      MXFP4 (adahop_iht_quant);
 *   3. the fused MXFP4 + BF16 GEMM: the residual product on FP4 matrix cores
 *      and the outlier product in bf16 (adahop_gemm_mx);
 *   4. the fused scatter-add of the outlier product into the result (inside
 *      adahop_gemm_mx's epilogue).
 * Fig. 5 routes each of a linear layer's three products (forward, input
 * gradient, weight gradient) by its operand pattern pair to IHT, OE-Left,
 * OE-Right or BF16 (adahop_route); adahop_gemm runs the whole path for one
 * product.
 *
 * Conventions
 *   - Every tensor pointer is a DEVICE pointer owned by the caller. The
 *     library never allocates, frees or synchronizes device memory; scratch
 *     space is the caller's workspace (adahop_detect_noalloc alone uses a
 *     static device array of the library instead). Every launch is enqueued
 *     on `stream` (a hipStream_t, NULL = the null stream) and the call
 *     returns at once.
 *   - bf16 tensors are uint16 bit patterns, row-major, leading dimension `ld`
 *     in elements (ld >= cols). A bf16 input quantized along its rows
 *     (contraction along columns) must have 16-byte aligned rows: base
 *     pointer 16-byte aligned and ld % 8 == 0. Packed code buffers must be
 *     16-byte aligned.
 *   - Textbook frame of a product: C[m,n] = A[m,K] * B[K,n], K the inner
 *     (contraction) dimension.
 *   - MXFP4 operand (OCP Microscaling v1.0 MXFP4): 4-bit E2M1 codes, two per
 *     byte, element 2j in the low nibble, stored [outer][K/2]; one E8M0 scale
 *     byte per 32 consecutive K-elements, stored [outer][K/32]. K runs
 *     contiguously. For A, outer = m (its rows); for B, outer = n (its
 *     columns).
 *   - Outlier index sets are int32, ascending, unique, on the device.
 *   - Errors: argument errors are found on the host before any launch and
 *     return ADAHOP_ERR_INVALID (or ADAHOP_ERR_UNSUPPORTED for a valid but
 *     unimplemented case) with a message in adahop_last_error(); a too-small
 *     workspace returns ADAHOP_ERR_WORKSPACE; a failed launch returns
 *     ADAHOP_ERR_HIP. Non-finite inputs are not supported (results
 *     unspecified). Outputs must not alias inputs.
 *   - Thread safety: calls on different streams may run concurrently;
 *     adahop_last_error() is per host thread.
 *   - adahop_gemm with OE_LEFT or OE_RIGHT quantizes the operand FOID does
 *     not scan beside FOID: in FOID's own launch when FOID's selection takes
 *     at most two levels (k <= 256, up to 16384 candidates at k = 64);
 *     otherwise, when the two operands exceed 96 MB of bf16, on a second
 *     stream the library creates once per device (default priority), forked
 *     from `stream` with an event and joined back before the GEMM;
 *     otherwise after FOID on `stream`. The call's completion stays ordered
 *     on `stream`.
 */
#ifndef ADAHOP_H
#define ADAHOP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ADAHOP_API __attribute__((visibility("default")))

typedef enum {
  ADAHOP_OK = 0,
  ADAHOP_ERR_INVALID = 1,     /* bad argument (detected before any launch) */
  ADAHOP_ERR_UNSUPPORTED = 2, /* valid but not implemented (alignment, sizes) */
  ADAHOP_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  ADAHOP_ERR_HIP = 4          /* a HIP runtime call or launch failed */
} adahop_status;

/* Outlier pattern of a stored tensor (Table 1's R / C / N). */
typedef enum { ADAHOP_PAT_NONE = 0, ADAHOP_PAT_ROW = 1, ADAHOP_PAT_COL = 2 } adahop_pattern;

/* The three products of a linear layer Y = X W^T (Table 1's columns):
 * FWD   Y  [T,Dout]    = X [T,Din] * W^T       (lhs X,  rhs W [Dout,Din])
 * DGRAD dX [T,Din]     = GY [T,Dout] * W       (lhs GY, rhs W [Dout,Din])
 * WGRAD dW [Dout,Din]  = GY^T * X              (lhs GY, rhs X [T,Din]) */
typedef enum { ADAHOP_OP_FWD = 0, ADAHOP_OP_DGRAD = 1, ADAHOP_OP_WGRAD = 2 } adahop_op;

/* Path of one product (Fig. 5). OE_INNER extracts inner-dimension lines of
 * both operands into a dense rank-k bf16 term; MXFP4 is plain quantization
 * without rotation or extraction (a baseline). */
typedef enum {
  ADAHOP_ROUTE_AUTO = -1,
  ADAHOP_ROUTE_BF16 = 0,
  ADAHOP_ROUTE_IHT = 1,
  ADAHOP_ROUTE_OE_LEFT = 2,
  ADAHOP_ROUTE_OE_RIGHT = 3,
  ADAHOP_ROUTE_OE_INNER = 4,
  ADAHOP_ROUTE_MXFP4 = 5
} adahop_route_t;

typedef enum { ADAHOP_AXIS_ROWS = 0, ADAHOP_AXIS_COLS = 1 } adahop_axis;
typedef enum { ADAHOP_OUT_BF16 = 0, ADAHOP_OUT_F32 = 1 } adahop_out_dtype;

/* Layout of packed MXFP4 operands in an adahop_gemm workspace.
 *   ROWS  : codes [outer][K/2], scales [outer][K/32] (as adahop_iht_quant).
 *   KCHUNK: K cut into chunks of 128: codes [K/128][outer][64] and scales
 *           [K/128][outer][4], i.e. chunk c of row r holds K-elements
 *           128 c .. 128 c + 127 of that row, each chunk of all rows
 *           contiguous -- the order in which the GEMM streams them. A
 *           chunk's four scale bytes are its blocks' in the order 0, 2, 1, 3. */
typedef enum { ADAHOP_LAYOUT_ROWS = 0, ADAHOP_LAYOUT_KCHUNK = 1 } adahop_layout;

ADAHOP_API const char* adahop_status_string(int status);
/* Detail of the last failure on this host thread ("" if none). */
ADAHOP_API const char* adahop_last_error(void);
ADAHOP_API int adahop_version(void);

/* ---------------------------------------------------------------------------
 * Routing (host only, pure). Fig. 5 routes each product by the pattern pair
 * of its operands; Fig. 2 and the abstract say IHT (mixing along the inner
 * dimension) suppresses outliers that lie along the inner dimension and not
 * those along the outer one. Rule, in the textbook frame: A is hurt if its
 * outlier lines are rows, B if its outlier lines are columns; neither -> IHT,
 * A only -> OE_LEFT, B only -> OE_RIGHT, both -> BF16. Patterns are given in
 * each tensor's storage frame (as in Table 1); a tensor used transposed swaps
 * ROW and COL. Returns ADAHOP_ROUTE_AUTO for an invalid op or pattern. */
ADAHOP_API adahop_route_t adahop_route(adahop_op op, adahop_pattern pat_lhs,
                                       adahop_pattern pat_rhs);

/* ---------------------------------------------------------------------------
 * Pattern calibration (Table 1 names the three patterns; Fig. 4 and Fig. 8
 * show them on real tensors, and the pages give no numeric test). Reading
 * used here: a tensor is Row-wise when a few rows carry far more energy than
 * the typical row, Column-wise likewise for columns, None otherwise,
 * measured with FOID's own line score.
 *
 * adahop_line_scores writes each line's FOID score (the probe variance
 * defined below for adahop_detect, bit for bit) to scores_out, a DEVICE
 * array of fp64 [rows] (axis ROWS) or [cols] (axis COLS). Enqueued on
 * `stream`; no workspace. Errors as adahop_detect's argument checks.
 *
 * adahop_classify_pattern (host only, pure) takes HOST copies of a tensor's
 * row scores and column scores and compares, per axis, r = max / median
 * (the median is the lower one: the element of rank (n - 1) / 2 in
 * ascending order): if the larger r is below `threshold` the pattern is
 * NONE, else ROW when r_rows >= r_cols and COL otherwise. A zero median with
 * a positive maximum counts as an infinite ratio; an all-zero axis as 1.
 * Returns ADAHOP_PAT_NONE for null pointers or empty arrays. */
ADAHOP_API adahop_status adahop_line_scores(const uint16_t* t, int64_t rows, int64_t cols,
                                            int64_t ld, adahop_axis axis, int32_t probe,
                                            double* scores_out, void* stream);
ADAHOP_API adahop_pattern adahop_classify_pattern(const double* row_scores, int64_t rows,
                                                  const double* col_scores, int64_t cols,
                                                  double threshold);

/* ---------------------------------------------------------------------------
 * FOID (appendix, kernel 1; Fig. 9). Candidates are the rows (axis ROWS:
 * statistics over t[r, 0:P]) or the columns (axis COLS: t[0:P, c]) of the
 * bf16 tensor t [rows, cols], P = min(probe, line length). Each candidate's
 * score is the population variance of those P values, computed in fp64 in
 * index order (sum, mean, then sum of squared deviations). The k candidates
 * with the largest score (ties: lower index first) are written to idx_out
 * (device int32[k]) in ascending order. Deterministic. Needs
 * adahop_detect_workspace_size(...) bytes of workspace: none up to 1024
 * candidates (4096 when k > 256), else the survivor lists of the selection
 * levels (k scores and indices per chunk of candidates: 256 or 512 when the
 * first level's survivors then fit in 1024 entries, else 1024, or 4096
 * when k > 256; two lists) and 256 bytes for a counter; ws may be NULL when
 * the size is 0.
 * Errors: INVALID if t/idx_out is NULL, rows/cols < 1, ld < cols, probe < 1,
 * k < 1 or k > number of candidates; UNSUPPORTED if k > 1024. */
ADAHOP_API size_t adahop_detect_workspace_size(int64_t rows, int64_t cols, adahop_axis axis,
                                               int32_t k);
ADAHOP_API adahop_status adahop_detect(const uint16_t* t, int64_t rows, int64_t cols,
                                       int64_t ld, adahop_axis axis, int32_t probe,
                                       int32_t k, int32_t* idx_out, void* ws,
                                       size_t ws_bytes, void* stream);

/* FOID without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Same arguments, checks and result as adahop_detect; the
 * selection's scratch (what adahop_detect_workspace_size reports) lives in a
 * static device array of adahop_detect_noalloc_max_bytes() bytes (1 MiB),
 * one per GPU, that the library holds until the process ends. The call
 * itself allocates nothing and clears what must start at zero with a kernel,
 * not a memset. Errors: as adahop_detect, and UNSUPPORTED when the
 * selection needs more scratch than that (e.g. k = 1024 over more than about
 * 170 000 candidates; k = 64 over more than about 1.4 million). Every call
 * on one GPU shares that GPU's array: calls that overlap in time on one GPU
 * (different streams or host threads without ordering) race and give
 * unspecified indices; order them on one stream. */
ADAHOP_API size_t adahop_detect_noalloc_max_bytes(void);
ADAHOP_API adahop_status adahop_detect_noalloc(const uint16_t* t, int64_t rows, int64_t cols,
                                               int64_t ld, adahop_axis axis, int32_t probe,
                                               int32_t k, int32_t* idx_out, void* stream);

/* ---------------------------------------------------------------------------
 * Zero + gather + IHT + MXFP4 quantization (appendix, kernel 2; abstract).
 * src is bf16 [rows, cols]. contract COLS: 32-blocks run along each row
 * (K = cols, outer = rows); contract ROWS: 32-blocks run down each column
 * (K = rows, outer = cols). K must be a multiple of 32.
 * Zeroing: the nzero lines zero_idx (device, ascending, unique) -- rows of
 * src if zero_axis is ROWS, columns if COLS -- are treated as +0 (the
 * residual with the outliers removed). gathered (device, may be NULL when
 * nzero > 0 and the lines are not needed) receives a compact bf16 copy of
 * those lines, one line per row: [nzero][cols] for rows, [nzero][rows] for
 * columns.
 * Rotation: hadamard_block 32 applies the orthonormal 32-point Walsh-Hadamard
 * transform (Sylvester order, fp32 butterflies with strides 1,2,4,8,16, then
 * one multiply by fp32(1/sqrt(32))) to each block; 0 applies none.
 * Quantization (OCP MX v1.0): scale exponent s = floor(log2(block amax)) - 2,
 * clamped to [-127, 127], stored as the byte s + 127 (0x00 for an all-zero
 * block); each element's code is the sign bit and the E2M1 magnitude nearest
 * to |y| / 2^s, ties to the even code, saturating at 6.
 * Output codes [outer][K/2] and scales [outer][K/32] (device).
 * Errors: INVALID for NULL src/codes/scales, bad sizes, K % 32 != 0,
 * hadamard_block not in {0, 32}, nzero < 0, or zero_idx NULL with nzero > 0;
 * UNSUPPORTED if codes or gathered are not 16-byte aligned, (contract COLS)
 * src rows are not 16-byte aligned, or nzero > 1024. Indices are not
 * validated on the device: unsorted or repeated zero_idx gives unspecified
 * results, out-of-range entries are ignored. */
ADAHOP_API adahop_status adahop_iht_quant(const uint16_t* src, int64_t rows, int64_t cols,
                                          int64_t ld, adahop_axis contract,
                                          int32_t hadamard_block, const int32_t* zero_idx,
                                          int32_t nzero, adahop_axis zero_axis,
                                          uint8_t* codes, uint8_t* scales, uint16_t* gathered,
                                          void* stream);

/* ---------------------------------------------------------------------------
 * Fused MXFP4 + BF16 GEMM with the scatter-add epilogue (appendix, kernels 3
 * and 4). */
typedef struct {
  const uint8_t* codes;   /* [outer][K/2] */
  const uint8_t* scales;  /* [outer][K/32] */
  int64_t outer;          /* m for A, n for B */
  int64_t K;
} adahop_mx_operand;

/* A bf16 factor of the outlier product, seen as [outer][inner]: element
 * (r, t) sits at ptr[r * ld + t] if inner_contiguous, else ptr[t * ld + r]. */
typedef struct {
  const uint16_t* ptr;
  int64_t ld;
  int32_t inner_contiguous;
  int32_t reserved;
} adahop_bf16_view;

/* The outlier (OE) term, P = a * b^T contracted over the views' inner index:
 *   OE_LEFT : a = the k extracted rows of A ([k][K]), b = B in bf16 ([n][K]);
 *             C[idx[p], j] += P[p][j].
 *   OE_RIGHT: a = A in bf16 ([m][K]), b = the k extracted columns of B
 *             ([k][K]); C[i, idx[p]] += P[i][p].
 *   OE_INNER: a = A's k extracted columns ([m][k]), b = B's k extracted rows
 *             ([n][k]); C[i, j] += P[i][j].
 * The add happens on fp32 values before the single rounding of C. */
typedef struct {
  adahop_route_t route;   /* OE_LEFT, OE_RIGHT or OE_INNER */
  int32_t k;
  const int32_t* idx;     /* device [k]; unused (may be NULL) for OE_INNER */
  adahop_bf16_view a;
  adahop_bf16_view b;
} adahop_oe;

/* C[m,n] (row-major, leading dim ldc, bf16 or fp32) = deq(A) * deq(B)^T with
 * fp32 accumulation, plus the OE term if oe != NULL. Needs
 * adahop_gemm_mx_workspace_size(...) bytes of 16-byte aligned workspace: the
 * outlier product's partial sums (OE_LEFT/OE_RIGHT) and, when K is a multiple
 * of 512, a copy of both scale arrays reordered for the GEMM plus, when the
 * last round of 256 x 256 tiles is split along K (at most half a round left
 * over from whole rounds of one tile per compute unit of the current device
 * -- 256 on an MI355X --, K / 128 a multiple of 8 and at least 32),
 * 256 KB of fp32 partial sums per tile part (0 when none applies; ws may then
 * be NULL). Its contents after the call are unspecified.
 * Errors: INVALID for NULL pointers, K mismatch, K % 32 != 0, ldc < n, a bad
 * out_dtype, bad OE descriptors; WORKSPACE for a missing or short workspace;
 * UNSUPPORTED for k > 1024, codes not 16-byte aligned or a misaligned
 * workspace. */
ADAHOP_API size_t adahop_gemm_mx_workspace_size(int64_t m, int64_t n, int64_t K,
                                                const adahop_oe* oe);
ADAHOP_API adahop_status adahop_gemm_mx(const adahop_mx_operand* A,
                                        const adahop_mx_operand* B, const adahop_oe* oe,
                                        void* C, int64_t ldc, adahop_out_dtype out_dtype,
                                        void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * One AdaHOP product end to end: route, FOID on the operand and axis the route
 * extracts, zero + gather + IHT + MXFP4 on both operands (along each one's
 * contraction axis), the fused GEMM and the scatter-add.
 *   FWD  : lhs X [T,Din],  rhs W [Dout,Din] -> out Y  [T,Dout]
 *   DGRAD: lhs GY [T,Dout], rhs W [Dout,Din] -> out dX [T,Din]
 *   WGRAD: lhs GY [T,Dout], rhs X [T,Din]    -> out dW [Dout,Din]
 * lhs, rhs and out are contiguous row-major. route AUTO applies adahop_route
 * to (pat_lhs, pat_rhs); oe_rank is the number of extracted lines (64 on the
 * pages, Fig. 10). The contraction length (Din, Dout or T) must be a
 * multiple of 32. The workspace holds, after the call, the quantized
 * operands and the outlier lines at the offsets adahop_gemm_plan reports;
 * the operands are in the plan's layout (KCHUNK when the contraction length
 * is a multiple of 512 and each packed operand is under 2 GiB, else ROWS).
 * Errors: as for the stage calls; INVALID for a bad op or route, or an OE
 * route with oe_rank < 1 or above the number of candidate lines.
 * Route BF16 (both operands hurt) computes the plain product on bf16 matrix
 * cores with fp32 accumulation and no packed operands (oe_rank is ignored).
 * When the contraction length is a multiple of 128 an operand not
 * contiguous along K (DGRAD: W; WGRAD: GY and X) is read in place if its
 * row length is a multiple of 8 and it is under 2 GiB; the workspace holds
 * K-major bf16 copies of the others, for a forward with 8192 or more rows on
 * one side a copy across K of the other operand (read faster that way), and
 * the fp32 parts of tiles split along K. Otherwise it needs none. With an
 * operand or the workspace not 16-byte aligned it runs on a slower tile
 * kernel instead. */
typedef struct {
  adahop_route_t route;   /* resolved route */
  int64_t m, n, K;        /* textbook-frame sizes */
  int32_t k;              /* extracted lines (0 without OE) */
  int32_t scan_tensor;    /* 0 = lhs, 1 = rhs, -1 = no FOID */
  adahop_axis scan_axis;  /* candidate lines: rows or columns of that tensor */
  adahop_layout layout;   /* layout of the packed operands below */
  size_t ws_bytes;        /* workspace the call needs */
  /* Byte offsets into the workspace (SIZE_MAX if absent): */
  size_t off_idx;         /* int32 [k] FOID indices */
  size_t off_a_codes, off_a_scales;   /* A packed (outer = m) in `layout` */
  size_t off_b_codes, off_b_scales;   /* B packed (outer = n) in `layout` */
  size_t off_lhs_lines;   /* bf16 lines gathered from lhs (layout as adahop_iht_quant) */
  size_t off_rhs_lines;   /* bf16 lines gathered from rhs */
  int32_t oe_in_quant;    /* 1: the outlier product is formed in the other operand's
                             quantization (asked for with adahop_gemm_options) */
} adahop_plan;

ADAHOP_API adahop_status adahop_gemm_plan(adahop_op op, int64_t T, int64_t Din, int64_t Dout,
                                          adahop_pattern pat_lhs, adahop_pattern pat_rhs,
                                          adahop_route_t route, int32_t oe_rank,
                                          adahop_plan* plan);
ADAHOP_API size_t adahop_gemm_workspace_size(adahop_op op, int64_t T, int64_t Din,
                                             int64_t Dout, adahop_pattern pat_lhs,
                                             adahop_pattern pat_rhs, adahop_route_t route,
                                             int32_t oe_rank);
ADAHOP_API adahop_status adahop_gemm(adahop_op op, const uint16_t* lhs, const uint16_t* rhs,
                                     int64_t T, int64_t Din, int64_t Dout,
                                     adahop_pattern pat_lhs, adahop_pattern pat_rhs,
                                     adahop_route_t route, int32_t oe_rank, void* out,
                                     adahop_out_dtype out_dtype, void* ws, size_t ws_bytes,
                                     void* stream);

/* Options of adahop_gemm_plan_ex and adahop_gemm_ex (NULL: all defaults,
 * which is adahop_gemm's behaviour). reserved must be zero.
 * oe_in_quant = 1: with OE_LEFT or OE_RIGHT, when the operand FOID does not
 * scan is quantized down its columns (contracted along its rows: DGRAD's W,
 * both WGRAD operands) and k <= 64, that operand's quantization also forms
 * the outer outlier product -- its rank-k product with the extracted lines,
 * fp32 partial sums per group of 128-row tiles, then their sum in group
 * order -- so the operand is read once (appendix, kernels 2 and 3: the
 * outlier product beside the quantization's single pass). The stages then
 * run one after another on `stream`: FOID, the scanned operand's
 * quantization (which gathers the lines), the other's with the partial
 * sums, their sum, the GEMM, whose epilogue adds the sum to the extracted
 * lines before the single rounding. The plan reports whether it applies
 * (plan.oe_in_quant); where it does not, the call runs as adahop_gemm. The
 * default path, which quantizes that operand beside FOID and forms the
 * outlier product inside the GEMM launch, measured faster on the workloads
 * here; this one exists for the one-read schedule and its measurement.
 * Errors: INVALID for oe_in_quant not 0 or 1 or a reserved field not 0;
 * otherwise as adahop_gemm_plan / adahop_gemm_timed (stage_events may be
 * NULL). */
typedef struct {
  int32_t oe_in_quant;
  int32_t reserved[7];
} adahop_gemm_options;

ADAHOP_API adahop_status adahop_gemm_plan_ex(adahop_op op, int64_t T, int64_t Din, int64_t Dout,
                                             adahop_pattern pat_lhs, adahop_pattern pat_rhs,
                                             adahop_route_t route, int32_t oe_rank,
                                             const adahop_gemm_options* opts,
                                             adahop_plan* plan);
ADAHOP_API adahop_status adahop_gemm_ex(adahop_op op, const uint16_t* lhs, const uint16_t* rhs,
                                        int64_t T, int64_t Din, int64_t Dout,
                                        adahop_pattern pat_lhs, adahop_pattern pat_rhs,
                                        adahop_route_t route, int32_t oe_rank,
                                        const adahop_gemm_options* opts, void* out,
                                        adahop_out_dtype out_dtype, void* ws, size_t ws_bytes,
                                        void* stream, void* const* stage_events);

/* ---------------------------------------------------------------------------
 * Saved forward context (appendix, kernel 2: for the activation of the
 * forward path, the quantized residual and the bf16 outlier tensor are kept
 * for backpropagation). The only backward product that reads the activation
 * X [T, Din] is the weight gradient dW = GY^T X, contracting over T, so the
 * context keeps X in the form that product consumes: the k columns its FOID
 * extracts (route OE_RIGHT), the residual with those columns zeroed, rotated
 * (FWHT-32, not for route MXFP4) and MXFP4-quantized along T, and those
 * columns in bf16 -- 17/32 bytes per element plus 2 k T for the lines, up to
 * 3.76x less than X in bf16. adahop_gemm_wgrad_ctx then computes the weight
 * gradient from GY and the context alone, bit for bit what adahop_gemm
 * (WGRAD, GY, X, ...) computes from X.
 *
 * pat_gy, pat_x, route and oe_rank are those of the weight gradient
 * (route AUTO applies adahop_route(WGRAD, pat_gy, pat_x)); the context
 * holds X for routes IHT, MXFP4 and OE_RIGHT. Routes BF16, OE_LEFT and
 * OE_INNER read X in bf16 in the backward (the outlier product of OE_LEFT
 * multiplies GY's lines by the whole of X) and return UNSUPPORTED.
 *
 * The context is one caller-owned device buffer of ctx_bytes (16-byte
 * aligned) at the plan's offsets: idx int32 [k] (SIZE_MAX without
 * extraction), codes and scales of X's residual with outer = Din, K = T in
 * the plan's layout (KCHUNK when T is a multiple of 512, as adahop_gemm's
 * weight gradient packs it), lines bf16 [k][T] (X's extracted columns, one
 * per row). adahop_ctx_save needs save_ws_bytes of workspace (FOID's
 * selection scratch; 0: ws may be NULL), adahop_gemm_wgrad_ctx
 * wgrad_ws_bytes (GY's packed form, the outlier product's partial sums and
 * the GEMM's scratch). Errors as adahop_gemm; INVALID for a context smaller
 * than its plan. stage_events: as adahop_gemm_timed (NULL for none); the FOID
 * and rhs stages are empty. */
typedef struct {
  adahop_route_t route;   /* the weight gradient's resolved route */
  int64_t T, Din, Dout;
  int32_t k;              /* extracted columns of X (0 without extraction) */
  adahop_layout layout;   /* layout of the kept codes and scales */
  size_t ctx_bytes;
  size_t off_idx, off_codes, off_scales, off_lines;   /* SIZE_MAX if absent */
  size_t save_ws_bytes;   /* workspace of adahop_ctx_save */
  size_t wgrad_ws_bytes;  /* workspace of adahop_gemm_wgrad_ctx */
} adahop_ctx_plan_t;

ADAHOP_API adahop_status adahop_ctx_plan(int64_t T, int64_t Din, int64_t Dout,
                                         adahop_pattern pat_gy, adahop_pattern pat_x,
                                         adahop_route_t route, int32_t oe_rank,
                                         adahop_ctx_plan_t* plan);
ADAHOP_API adahop_status adahop_ctx_save(const uint16_t* X, int64_t T, int64_t Din,
                                         int64_t Dout, adahop_pattern pat_gy,
                                         adahop_pattern pat_x, adahop_route_t route,
                                         int32_t oe_rank, void* ctx, size_t ctx_bytes,
                                         void* ws, size_t ws_bytes, void* stream);
ADAHOP_API adahop_status adahop_gemm_wgrad_ctx(const uint16_t* GY, const void* ctx,
                                               size_t ctx_bytes, int64_t T, int64_t Din,
                                               int64_t Dout, adahop_pattern pat_gy,
                                               adahop_pattern pat_x, adahop_route_t route,
                                               int32_t oe_rank, void* out,
                                               adahop_out_dtype out_dtype, void* ws,
                                               size_t ws_bytes, void* stream,
                                               void* const* stage_events);

/* As adahop_gemm, and if stage_events is not NULL it must hold
 * ADAHOP_STAGE_EVENTS created hipEvent_t handles: events[0] is recorded on
 * `stream` before the first launch and events[1..6] after the FOID, lhs
 * quantization, rhs quantization (which ends with reordering both scale
 * arrays for the GEMM), outlier product, GEMM main kernel and GEMM tail
 * stages (a stage that does not run records its event right after the
 * previous one). The tail is what finishes the main kernel's output: the
 * fixup of a split last round of tiles and, when the outlier product ran
 * inside the main kernel, its scatter into the extracted lines. With
 * OE_LEFT and OE_RIGHT the operand FOID does not scan is quantized in
 * FOID's launch (the FOID stage then holds both, and that operand's stage is
 * empty), on a second stream (its stage is empty here, the ROWS-layout scale
 * reordering falls in the GEMM stage, and the other stages overlap with it)
 * or in its own stage after FOID, as the notes at the top say. With route
 * BF16 the lhs and rhs stages are the operands' K-major copies, if any.
 * With the outlier product formed in the quantization (adahop_gemm_ex,
 * oe_in_quant), the stages follow that order: with OE_RIGHT the lhs stage is
 * empty and the lhs's quantization with the partial sums falls in the
 * outlier product's stage, with their sum. */
#define ADAHOP_STAGE_EVENTS 7
ADAHOP_API adahop_status adahop_gemm_timed(adahop_op op, const uint16_t* lhs,
                                           const uint16_t* rhs, int64_t T, int64_t Din,
                                           int64_t Dout, adahop_pattern pat_lhs,
                                           adahop_pattern pat_rhs, adahop_route_t route,
                                           int32_t oe_rank, void* out,
                                           adahop_out_dtype out_dtype, void* ws,
                                           size_t ws_bytes, void* stream,
                                           void* const* stage_events);

#ifdef __cplusplus
}
#endif
#endif /* ADAHOP_H */
