/*
 * AdaHOP oracle (CPU, plain C11, built with -ffp-contract=off).
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU baseline, never by the product path. Shares no code with the
 * GPU library.
 *
 * Each function states the passage of "AdaHOP: Fast and Accurate Low-Precision
 * Training via Outlier-Pattern-Aware Rotation" (arXiv 2604.02525) it follows,
 * and the reading taken where that passage leaves a detail open.
 */
#include "adahop_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int adahop_ref_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ------------------------------------------------------------------------ */
/* Routing. Abstract: IHT where mixing along the inner dimension suppresses  */
/* the operands' outliers, OE (one operand's dominant outlier lines moved to */
/* a high-precision path) where it does not. Fig. 2: a Hadamard applied along */
/* rows (on the right) flattens Column-wise outliers, one along columns does */
/* not. Fig. 5: each of a layer's three products takes IHT, OE-Left,         */
/* OE-Right or BF16 by its pattern pair. The figure's table itself is not    */
/* legible, so the rule below is derived from those facts:                   */
/*   in C = A*B the rotation runs along A's columns and B's rows; A is hurt   */
/*   (outlier lines along the outer dim) iff it is Row-wise in that frame, B  */
/*   iff it is Column-wise. Neither hurt -> IHT; only A -> OE_LEFT; only B -> */
/*   OE_RIGHT; both -> BF16. Patterns arrive in each tensor's storage frame   */
/*   (as in Table 1); a tensor used transposed swaps Row and Column.          */
/* Parity unpinned beyond the products the pages configure: those cells and  */
/* Table 1's pair counts pin it; the rest of the table is this derivation.    */
/* ------------------------------------------------------------------------ */
static int swap_rc(int p) {
  return p == REF_PAT_ROW ? REF_PAT_COL : (p == REF_PAT_COL ? REF_PAT_ROW : p);
}

int adahop_ref_route(int op, int pat_lhs, int pat_rhs) {
  if (pat_lhs < 0 || pat_lhs > 2 || pat_rhs < 0 || pat_rhs > 2) return -1;
  int a, b; /* textbook-frame patterns */
  switch (op) {
    case REF_OP_FWD:   a = pat_lhs;          b = swap_rc(pat_rhs); break; /* X * W^T   */
    case REF_OP_DGRAD: a = pat_lhs;          b = pat_rhs;          break; /* GY * W    */
    case REF_OP_WGRAD: a = swap_rc(pat_lhs); b = pat_rhs;          break; /* GY^T * X  */
    default: return -1;
  }
  int a_hurt = (a == REF_PAT_ROW), b_hurt = (b == REF_PAT_COL);
  if (!a_hurt && !b_hurt) return REF_ROUTE_IHT;
  if (a_hurt && !b_hurt) return REF_ROUTE_OE_LEFT;
  if (!a_hurt && b_hurt) return REF_ROUTE_OE_RIGHT;
  return REF_ROUTE_BF16;
}

/* OE_LEFT extracts rows of A, OE_RIGHT columns of B, OE_INNER the inner lines
 * (A's columns, found on the lhs). Mapped back to the stored tensors:
 *   FWD   A = X,    B = W^T : A rows = X rows,  B cols = W rows,  A cols = X cols
 *   DGRAD A = GY,   B = W   : A rows = GY rows, B cols = W cols,  A cols = GY cols
 *   WGRAD A = GY^T, B = X   : A rows = GY cols, B cols = X cols,  A cols = GY rows */
int adahop_ref_scan_target(int op, int route, int* tensor, int* axis) {
  if (op < 0 || op > 2) return -1;
  if (route == REF_ROUTE_OE_LEFT) {
    *tensor = 0;
    *axis = op == REF_OP_WGRAD ? REF_AXIS_COLS : REF_AXIS_ROWS;
  } else if (route == REF_ROUTE_OE_RIGHT) {
    *tensor = 1;
    *axis = op == REF_OP_FWD ? REF_AXIS_ROWS : REF_AXIS_COLS;
  } else if (route == REF_ROUTE_OE_INNER) {
    *tensor = 0;
    *axis = op == REF_OP_WGRAD ? REF_AXIS_ROWS : REF_AXIS_COLS;
  } else {
    return -1;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* FOID (appendix, kernel 1; Fig. 9): each candidate row or column is scored */
/* by the variance of its first 64 elements; the k best become the outlier   */
/* lines, and their entries are zeroed in the residual.                      */
/* Readings: population variance (divide by P), two passes in fp64, summed   */
/* in index order; P = min(probe, line length); ties go to the lower index;  */
/* the k indices are returned in ascending order.                            */
/* ------------------------------------------------------------------------ */
typedef struct { double var; int64_t idx; } cand_t;

static int cand_cmp(const void* p, const void* q) {
  const cand_t* x = (const cand_t*)p;
  const cand_t* y = (const cand_t*)q;
  if (x->var > y->var) return -1;
  if (x->var < y->var) return 1;
  return (x->idx > y->idx) - (x->idx < y->idx);
}

static int i32_cmp(const void* p, const void* q) {
  int32_t x = *(const int32_t*)p, y = *(const int32_t*)q;
  return (x > y) - (x < y);
}

int adahop_ref_foid(const uint16_t* t, int64_t rows, int64_t cols, int64_t ld, int axis,
                    int probe, int k, int32_t* idx_out, double* var_out) {
  if (!t || !idx_out || rows < 1 || cols < 1 || ld < cols || probe < 1) return -1;
  if (axis != REF_AXIS_ROWS && axis != REF_AXIS_COLS) return -1;
  int64_t ncand = axis == REF_AXIS_ROWS ? rows : cols;
  int64_t len = axis == REF_AXIS_ROWS ? cols : rows;
  if (k < 1 || k > ncand) return -1;
  int64_t P = probe < len ? probe : len;
  cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)ncand);
  if (!c) return -1;
  for (int64_t l = 0; l < ncand; ++l) {
    double sum = 0.0;
    for (int64_t i = 0; i < P; ++i) {
      uint16_t h = axis == REF_AXIS_ROWS ? t[l * ld + i] : t[i * ld + l];
      sum += (double)bf16_to_f32(h);
    }
    double mean = sum / (double)P;
    double ss = 0.0;
    for (int64_t i = 0; i < P; ++i) {
      uint16_t h = axis == REF_AXIS_ROWS ? t[l * ld + i] : t[i * ld + l];
      double d = (double)bf16_to_f32(h) - mean;
      ss += d * d;
    }
    c[l].var = ss / (double)P;
    c[l].idx = l;
    if (var_out) var_out[l] = c[l].var;
  }
  qsort(c, (size_t)ncand, sizeof(cand_t), cand_cmp);
  for (int i = 0; i < k; ++i) idx_out[i] = (int32_t)c[i].idx;
  qsort(idx_out, (size_t)k, sizeof(int32_t), i32_cmp);
  free(c);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* IHT (abstract; appendix, kernel 2): a 1-D fast Walsh-Hadamard transform   */
/* over blocks of 32 along the inner dimension, applied to the residual.     */
/* Readings: orthonormal (Sylvester H_32 divided by sqrt(32)) so that the    */
/* product is unchanged in exact arithmetic, no random signs; fp32, the      */
/* standard butterfly with strides 1, 2, 4, 8, 16 in that order, each output */
/* (a + b, a - b) one rounded fp32 operation, then one rounded multiply by   */
/* fp32(1/sqrt(32)).                                                         */
/* ------------------------------------------------------------------------ */
void adahop_ref_fwht32(float y[32]) {
  for (int h = 1; h < 32; h <<= 1) {
    for (int i = 0; i < 32; ++i) {
      if (i & h) continue;
      float a = y[i], b = y[i + h];
      y[i] = a + b;
      y[i + h] = a - b;
    }
  }
  const float inv_sqrt32 = (float)(1.0 / sqrt(32.0));
  for (int i = 0; i < 32; ++i) y[i] = y[i] * inv_sqrt32;
}

/* ------------------------------------------------------------------------ */
/* MXFP4 (abstract; appendix, kernel 2: one scale per 32-element block along */
/* the inner dimension). The pages give no formula; the OCP MX v1.0 rule is  */
/* used: shared exponent = floor(log2(amax)) - 2 (2 = largest E2M1 exponent),*/
/* stored as E8M0 with bias 127 and clamped to [-127, 127]; an all-zero      */
/* block stores 0x00. Elements round to nearest E2M1 value, ties to the even */
/* code, saturating at 6; the sign bit is kept (so -tiny gives code 0x8).    */
/* ------------------------------------------------------------------------ */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

int adahop_ref_e2m1_magnitude(double v) {
  /* Midpoints between grid neighbours; at an exact midpoint the even code
   * (0, 2, 4, 6) wins, which makes the comparison <= or < alternate. */
  if (v <= 0.25) return 0;
  if (v < 0.75) return 1;
  if (v <= 1.25) return 2;
  if (v < 1.75) return 3;
  if (v <= 2.5) return 4;
  if (v < 3.5) return 5;
  if (v <= 5.0) return 6;
  return 7;
}

double adahop_ref_e2m1_value(int code) {
  double m = E2M1_GRID[code & 7];
  return (code & 8) ? -m : m;
}

void adahop_ref_mx_block(const float y[32], uint8_t codes[16], uint8_t* scale) {
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) {
    float a = fabsf(y[i]);
    if (a > amax) amax = a;
  }
  int s = 0;
  if (amax == 0.0f) {
    *scale = 0;
    s = -127;
  } else {
    int e;
    frexp((double)amax, &e);   /* amax = f * 2^e, f in [0.5, 1) */
    s = (e - 1) - 2;           /* floor(log2 amax) - 2 */
    if (s < -127) s = -127;
    if (s > 127) s = 127;
    *scale = (uint8_t)(s + 127);
  }
  memset(codes, 0, 16);
  for (int i = 0; i < 32; ++i) {
    double v = ldexp(fabs((double)y[i]), -s);
    int m = adahop_ref_e2m1_magnitude(v);
    int code = (signbit(y[i]) ? 8 : 0) | m;
    codes[i / 2] |= (uint8_t)(code << (4 * (i & 1)));
  }
}

/* ------------------------------------------------------------------------ */
/* Zero + gather + IHT + quantize over a whole tensor (appendix, kernels 1-2) */
/* ------------------------------------------------------------------------ */
static int in_sorted(const int32_t* idx, int32_t n, int64_t v) {
  int32_t lo = 0, hi = n;
  while (lo < hi) {
    int32_t mid = lo + (hi - lo) / 2;
    if (idx[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo < n && idx[lo] == v;
}

int adahop_ref_iht_quant(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld,
                         int contract, int hadamard_block, const int32_t* zero_idx,
                         int32_t nzero, int zero_axis, uint8_t* codes, uint8_t* scales,
                         uint16_t* gathered) {
  if (!src || !codes || !scales || rows < 1 || cols < 1 || ld < cols) return -1;
  if (contract != REF_AXIS_ROWS && contract != REF_AXIS_COLS) return -1;
  if (hadamard_block != 0 && hadamard_block != 32) return -1;
  if (nzero < 0 || (nzero > 0 && !zero_idx)) return -1;
  if (nzero > 0 && zero_axis != REF_AXIS_ROWS && zero_axis != REF_AXIS_COLS) return -1;
  int64_t K = contract == REF_AXIS_COLS ? cols : rows;
  int64_t outer = contract == REF_AXIS_COLS ? rows : cols;
  if (K % 32 != 0) return -1;
  int64_t zdim = zero_axis == REF_AXIS_ROWS ? rows : cols;
  for (int32_t i = 0; i < nzero; ++i) {
    if (zero_idx[i] < 0 || zero_idx[i] >= zdim) return -1;
    if (i > 0 && zero_idx[i] <= zero_idx[i - 1]) return -1; /* ascending, unique */
  }
  int64_t nblk = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t o = 0; o < outer; ++o) {
    for (int64_t b = 0; b < nblk; ++b) {
      float y[32];
      for (int j = 0; j < 32; ++j) {
        int64_t r = contract == REF_AXIS_COLS ? o : b * 32 + j;
        int64_t c = contract == REF_AXIS_COLS ? b * 32 + j : o;
        int zeroed = nzero > 0 && in_sorted(zero_idx, nzero, zero_axis == REF_AXIS_ROWS ? r : c);
        y[j] = zeroed ? 0.0f : bf16_to_f32(src[r * ld + c]);
      }
      if (hadamard_block == 32) adahop_ref_fwht32(y);
      adahop_ref_mx_block(y, codes + o * (K / 2) + b * 16, scales + o * nblk + b);
    }
  }
  if (gathered && nzero > 0) {
    /* One extracted line per row of `gathered`, in the source's order. */
    if (zero_axis == REF_AXIS_ROWS) {
      for (int32_t p = 0; p < nzero; ++p)
        for (int64_t c = 0; c < cols; ++c) gathered[p * cols + c] = src[zero_idx[p] * ld + c];
    } else {
      for (int32_t p = 0; p < nzero; ++p)
        for (int64_t r = 0; r < rows; ++r) gathered[p * rows + r] = src[r * ld + zero_idx[p]];
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Product of the dequantized operands (appendix, kernel 3: the residual     */
/* multiplication in MXFP4). C[i][j] = sum over 32-blocks b of               */
/* 2^(sA + sB) * (sum over the block of e2m1(a) * e2m1(b)). Each block sum is */
/* a multiple of 1/4 below 1152 in magnitude, hence exact in fp64; the sum   */
/* over blocks runs in block order.                                          */
/* ------------------------------------------------------------------------ */
static double code_at(const uint8_t* row, int64_t t) {
  uint8_t byte = row[t / 2];
  return adahop_ref_e2m1_value((t & 1) ? (byte >> 4) : (byte & 15));
}

int adahop_ref_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales,
                       const uint8_t* b_codes, const uint8_t* b_scales, int64_t K,
                       const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                       double* C, double* absC) {
  if (!a_codes || !a_scales || !b_codes || !b_scales || !rows || !cols || !C) return -1;
  if (K < 32 || K % 32 != 0 || nrows < 0 || ncols < 0) return -1;
  int64_t nblk = K / 32;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t a = 0; a < nrows; ++a) {
    const uint8_t* ar = a_codes + rows[a] * (K / 2);
    const uint8_t* as = a_scales + rows[a] * nblk;
    for (int64_t bcol = 0; bcol < ncols; ++bcol) {
      const uint8_t* br = b_codes + cols[bcol] * (K / 2);
      const uint8_t* bs = b_scales + cols[bcol] * nblk;
      double acc = 0.0, aacc = 0.0;
      for (int64_t blk = 0; blk < nblk; ++blk) {
        double s = 0.0, sa = 0.0;
        for (int64_t t = blk * 32; t < blk * 32 + 32; ++t) {
          double p = code_at(ar, t) * code_at(br, t);
          s += p;
          sa += fabs(p);
        }
        double scale = ldexp(1.0, ((int)as[blk] - 127) + ((int)bs[blk] - 127));
        acc += s * scale;
        aacc += sa * scale;
      }
      C[a * ncols + bcol] = acc;
      if (absC) absC[a * ncols + bcol] = aacc;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Product of bf16 operands in fp64: the high-precision outlier path         */
/* (abstract; appendix, kernel 3) and the BF16 route (Fig. 5).               */
/* ------------------------------------------------------------------------ */
int adahop_ref_gemm_bf16(const uint16_t* a, int64_t lda, int a_trans,
                         const uint16_t* b, int64_t ldb, int b_trans, int64_t K,
                         const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                         double* C, double* absC) {
  if (!a || !b || !rows || !cols || !C || K < 0 || nrows < 0 || ncols < 0) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t x = 0; x < nrows; ++x) {
    int64_t i = rows[x];
    for (int64_t y = 0; y < ncols; ++y) {
      int64_t j = cols[y];
      double acc = 0.0, aacc = 0.0;
      for (int64_t t = 0; t < K; ++t) {
        double av = bf16_to_f32(a_trans ? a[t * lda + i] : a[i * lda + t]);
        double bv = bf16_to_f32(b_trans ? b[j * ldb + t] : b[t * ldb + j]);
        double p = av * bv;   /* exact: two 8-bit significands */
        acc += p;
        aacc += fabs(p);
      }
      C[x * ncols + y] = acc;
      if (absC) absC[x * ncols + y] = aacc;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Running-error terms of an fp32 accumulation (test tolerance, not part of   */
/* the method). An accumulator that adds the products of a contraction in     */
/* index order, `step` at a time, rounds after each addition, so its error is */
/* at most u times the sum of the magnitudes of the partial sums it holds     */
/* (first order, Higham, "Accuracy and Stability of Numerical Algorithms",    */
/* recursive summation). With S_j the exact partial sum of the first j*step   */
/* products and R_j = max over i <= j of |S_i|:                               */
/*   walk = sum over j of (|S_j| + R_j),  rmax = R at the last j.             */
/* A run that starts over at some earlier position s (the contraction cut     */
/* into contiguous parts that are added afterwards) holds S_j - S_s, and      */
/* |S_j - S_s| <= |S_j| + R_j: walk bounds its partial sums as well.          */
/* ------------------------------------------------------------------------ */
static void walk_terms(const double* prod, int64_t K, int64_t step, double* walk, double* rmax) {
  double s = 0.0, w = 0.0, r = 0.0;
  for (int64_t t0 = 0; t0 < K; t0 += step) {
    int64_t t1 = t0 + step < K ? t0 + step : K;
    for (int64_t t = t0; t < t1; ++t) s += prod[t];
    double as = fabs(s);
    if (as > r) r = as;
    w += as + r;
  }
  *walk = w;
  *rmax = r;
}

int adahop_ref_walk_mx(const uint8_t* a_codes, const uint8_t* a_scales,
                       const uint8_t* b_codes, const uint8_t* b_scales, int64_t K, int64_t step,
                       const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                       double* walk, double* rmax) {
  if (!a_codes || !a_scales || !b_codes || !b_scales || !rows || !cols || !walk || !rmax) return -1;
  if (K < 32 || K % 32 != 0 || step < 1 || nrows < 0 || ncols < 0) return -1;
  int64_t nblk = K / 32;
#pragma omp parallel
  {
    double* prod = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(dynamic, 1)
    for (int64_t a = 0; a < nrows; ++a) {
      const uint8_t* ar = a_codes + rows[a] * (K / 2);
      const uint8_t* as = a_scales + rows[a] * nblk;
      for (int64_t bcol = 0; bcol < ncols; ++bcol) {
        const uint8_t* br = b_codes + cols[bcol] * (K / 2);
        const uint8_t* bs = b_scales + cols[bcol] * nblk;
        for (int64_t t = 0; t < K; ++t)
          prod[t] = code_at(ar, t) * code_at(br, t) *
                    ldexp(1.0, ((int)as[t / 32] - 127) + ((int)bs[t / 32] - 127));
        walk_terms(prod, K, step, &walk[a * ncols + bcol], &rmax[a * ncols + bcol]);
      }
    }
    free(prod);
  }
  return 0;
}

int adahop_ref_walk_bf16(const uint16_t* a, int64_t lda, int a_trans,
                         const uint16_t* b, int64_t ldb, int b_trans, int64_t K, int64_t step,
                         const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                         double* walk, double* rmax) {
  if (!a || !b || !rows || !cols || !walk || !rmax || K < 0 || step < 1 || nrows < 0 || ncols < 0)
    return -1;
#pragma omp parallel
  {
    double* prod = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t x = 0; x < nrows; ++x) {
      int64_t i = rows[x];
      for (int64_t y = 0; y < ncols; ++y) {
        int64_t j = cols[y];
        for (int64_t t = 0; t < K; ++t)
          prod[t] = (double)bf16_to_f32(a_trans ? a[t * lda + i] : a[i * lda + t]) *
                    (double)bf16_to_f32(b_trans ? b[j * ldb + t] : b[t * ldb + j]);
        walk_terms(prod, K, step, &walk[x * ncols + y], &rmax[x * ncols + y]);
      }
    }
    free(prod);
  }
  return 0;
}

int adahop_ref_dequant(const uint8_t* codes, const uint8_t* scales, int64_t outer, int64_t K,
                       double* out) {
  if (!codes || !scales || !out || outer < 0 || K % 32 != 0) return -1;
  for (int64_t o = 0; o < outer; ++o)
    for (int64_t t = 0; t < K; ++t)
      out[o * K + t] = ldexp(code_at(codes + o * (K / 2), t),
                             (int)scales[o * (K / 32) + t / 32] - 127);
  return 0;
}
