// Internal declarations of the AdaHOP HIP library (gfx950). Not installed.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/adahop.h"

namespace adahop {

// Per-thread error detail, set by fail().
void set_error(const std::string& msg);
adahop_status fail(adahop_status st, const std::string& msg);
adahop_status check_launch(const char* what);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
constexpr size_t kAlign = 256;
constexpr int kMaxK = 1024;  // largest outlier rank (FOID top-k, OE lines)

// ---- FOID -----------------------------------------------------------------
size_t foid_workspace_bytes(int64_t ncand, int32_t k);
// Whether foid_launch's grid fits (false: it would return UNSUPPORTED).
bool foid_fits(int64_t ncand, int32_t k);
// FOID's score of every candidate line, fp64 [ncand], on the device.
adahop_status line_scores_launch(const uint16_t* t, int64_t rows, int64_t cols, int64_t ld, int axis,
                                 int32_t probe, double* out, hipStream_t stream);
// The quantization (IHT over blocks of 32, MXFP4) of an operand with no
// extracted lines that FOID may run in its own launch. contract ROWS (blocks
// down the columns): src [K][outer]; contract COLS (blocks along the rows):
// src [outer][K]; row stride ld; codes and scales as iht_quant_launch writes
// them for that layout; stream_src as there.
struct QuantBeside {
  const uint16_t* src;
  int64_t K, outer, ld;
  uint8_t* codes;
  uint8_t* scales;
  int layout;
  int contract;
  bool stream_src;
};
// Whether FOID's selection over ncand candidates fits one launch of
// 256-thread workgroups (k <= 256, at most two levels) that also runs q's
// quantization (q suits the vectorized quantizer tiles of its direction).
bool foid_beside_fits(int64_t ncand, int32_t k, const QuantBeside& q);
// With `beside` and foid_beside_fits, the selection's workgroups and that
// quantization's share one launch and *beside_done is set; otherwise FOID
// runs as without it and the caller quantizes the operand itself.
adahop_status foid_launch(const uint16_t* t, int64_t rows, int64_t cols, int64_t ld, int axis,
                          int32_t probe, int32_t k, int32_t* idx_out, void* ws, size_t ws_bytes,
                          hipStream_t stream, const QuantBeside* beside = nullptr,
                          bool* beside_done = nullptr);

// ---- zero + gather + IHT + MXFP4 ------------------------------------------
// Whether iht_quant_launch's grid fits (false: it would return UNSUPPORTED).
bool iht_quant_fits(int64_t rows, int64_t cols, int contract);
// stream_src: load the source non-temporally (it is read once); false keeps
// it in the caches for a kernel that reads it again soon after (the outer
// outlier product's wide factor).
adahop_status iht_quant_launch(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld,
                               int contract, int32_t hadamard_block, const int32_t* zero_idx,
                               int32_t nzero, int zero_axis, uint8_t* codes, uint8_t* scales,
                               uint16_t* gathered, int layout, hipStream_t stream,
                               bool stream_src = true);

// The one-read variant of OE_LEFT / OE_RIGHT: the operand FOID does not scan,
// quantized down its columns (contract ROWS, K = rows), also forms the outer
// outlier product's partial sums P_s = (its columns) x lines^T over group s
// of K, fp32, in `partials` ([groups][cols][k], or [groups][k][cols] with
// by_line), from the k extracted lines ([k][K] bf16, 16-byte aligned).
// iht_quant_oe_groups returns the number of groups (0 if k > 64 or the
// sizes do not fit).
int iht_quant_oe_groups(int64_t K, int64_t outer, int32_t k, int* tiles_per_wg);
adahop_status iht_quant_oe_launch(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld,
                                  uint8_t* codes, uint8_t* scales, int layout,
                                  const uint16_t* lines, int32_t k, int by_line, float* partials,
                                  hipStream_t stream);

// ---- outlier product (bf16 MFMA) ------------------------------------------
// P_s[x][y] = sum over t in split s of X(x, t) * Y(y, t), fp32, for s < splits,
// laid out [splits][nx][ny] in `partials`, followed by their sum P [nx][ny]
// (so `partials` holds (splits + 1) * nx * ny floats).
struct Bf16View {
  const uint16_t* ptr;
  int64_t ld;
  int inner_contiguous;
};
int oe_splits(int64_t nx, int64_t ny, int64_t K);
// Whether the outlier product's grid fits (false: oe_product_launch would
// return UNSUPPORTED).
bool oe_product_fits(int64_t nx, int64_t ny);
adahop_status oe_product_launch(Bf16View X, Bf16View Y, int64_t nx, int64_t ny, int64_t K,
                                int splits, float* partials, hipStream_t stream);
// P = sum over s < splits of partials[s] (each `count` floats), in the order
// s = 0, 1, ..., written right after the partials.
adahop_status oe_reduce_launch(float* partials, int splits, int64_t count, hipStream_t stream);
// Full bf16 product written to C (the BF16 route): C[i][j] = sum_t X(i,t) Y(j,t).
adahop_status bf16_gemm_launch(Bf16View X, Bf16View Y, int64_t m, int64_t n, int64_t K,
                               void* C, int64_t ldc, int out_f32, hipStream_t stream);
// The same product on the FP4 GEMM's ring kernel with bf16 matrix cores,
// K % 128 == 0 (bf16_ring_ok). Each operand is 16-byte aligned and either
// along K (a [m, K] row-major, row stride K) or, with *_across, stored
// across K (a [K, lda] row-major holding a(i, t) at t * lda + i; lda % 8 ==
// 0 and under 2 GiB: bf16_ring_across_ok). `scratch` holds
// bf16_ring_scratch_bytes(m, n, K) bytes (the split tiles' fp32 parts,
// 16-byte aligned).
bool bf16_ring_ok(int64_t m, int64_t n, int64_t K);
bool bf16_ring_across_ok(int64_t K, int64_t ld);
size_t bf16_ring_scratch_bytes(int64_t m, int64_t n, int64_t K);
adahop_status bf16_ring_launch(const uint16_t* a, int a_across, int64_t lda, const uint16_t* b,
                               int b_across, int64_t ldb, int64_t m, int64_t n, int64_t K, void* C,
                               int64_t ldc, int out_f32, void* scratch, size_t scratch_bytes,
                               hipStream_t stream, hipEvent_t main_done = nullptr);
// dst [cols, rows] (leading dim rows) = transpose of src [rows, cols]
// (leading dim ld).
adahop_status bf16_transpose_launch(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld,
                                    uint16_t* dst, hipStream_t stream);
bool bf16_transpose_fits(int64_t rows, int64_t cols);

// ---- FP4 GEMM with the OE epilogue ----------------------------------------
struct OeEpilogue {
  int mode;                 // 0 none, ADAHOP_ROUTE_OE_LEFT / _OE_RIGHT / _OE_INNER
  int32_t k;
  const int32_t* idx;       // OE_LEFT / OE_RIGHT
  const float* partials;    // OE_LEFT: [splits][k][n]; OE_RIGHT: [splits][m][k]; then P
  int splits;
  Bf16View a, b;            // OE_INNER factors: a [m][k], b [n][k]; OE_LEFT / OE_RIGHT:
                            // the outlier product's factors, as for oe_product_launch
  // OE_LEFT / OE_RIGHT computed inside the GEMM launch (fused_parts > 0, from
  // oe_fused_parts): `fused_ws` holds oe_fused_bytes(...) bytes, 16-byte
  // aligned, for the partial sums and the extracted lines' residual.
  int fused_parts;
  float* fused_ws;
};
// K-parts of the outer outlier product (OE_LEFT / OE_RIGHT, X = a, Y = b as
// in oe_product_launch) when it runs as work items of the main GEMM kernel,
// or 0 when it runs as oe_product_kernel before the GEMM: k <= 64, the main
// kernel applies to (m, n, K), the wide factor (a for OE_RIGHT, b for
// OE_LEFT) is stored across K with a row of a multiple of 8 elements under
// 2 GiB, the lines (the other factor) run along K in rows of a multiple of 8
// elements; with check_ptrs, both 16-byte aligned.
int oe_fused_parts(int64_t m, int64_t n, int64_t K, int mode, int32_t k, Bf16View a, Bf16View b,
                   bool check_ptrs);
// Whether gemm_mx_launch runs the main (ring) kernel for these operands.
bool gemm_mx_ring_used(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                       const uint8_t* b_scales, int64_t m, int64_t n, int64_t K, int layout);
// Workspace of the fused outlier product: parts x wide x k partial sums plus
// wide x k residuals, fp32.
size_t oe_fused_bytes(int64_t m, int64_t n, int mode, int32_t k, int parts);
// Workspace the GEMM needs for (m, n, K) in `layout`, when the main kernel
// applies (K % 512 == 0), else 0: for ROWS, stage-major copies of both scale
// arrays ([K/128][rows] words; gemm_mx_stage_scales writes them), then, for
// both layouts, the fp32 parts of the tiles the main kernel splits along K
// in its last round (256 KB per part).
size_t gemm_mx_scratch_bytes(int64_t m, int64_t n, int64_t K, int layout);
// Whether (m, n, K) operands may be packed K-chunked (ADAHOP_LAYOUT_KCHUNK):
// the main kernel applies and stage offsets fit 31 bits.
bool gemm_mx_kchunk_ok(int64_t m, int64_t n, int64_t K);
// Whether the GEMM's tile count fits (false: gemm_mx_launch would return
// UNSUPPORTED).
bool gemm_mx_fits(int64_t m, int64_t n);
adahop_status gemm_mx_stage_scales(const uint8_t* a_codes, const uint8_t* a_scales,
                                   const uint8_t* b_codes, const uint8_t* b_scales, int64_t m,
                                   int64_t n, int64_t K, void* scratch, size_t scratch_bytes,
                                   hipStream_t stream);
// layout ROWS: scales reordered by gemm_mx_stage_scales into `scratch` when
// the main kernel applies; KCHUNK: operands as ADAHOP_LAYOUT_KCHUNK. `scratch`
// holds gemm_mx_scratch_bytes(m, n, K, layout) bytes.
adahop_status gemm_mx_launch(const uint8_t* a_codes, const uint8_t* a_scales,
                             const uint8_t* b_codes, const uint8_t* b_scales, int64_t m,
                             int64_t n, int64_t K, int layout, const OeEpilogue& oe, void* C,
                             int64_t ldc, int out_f32, void* scratch, size_t scratch_bytes,
                             hipStream_t stream, hipEvent_t main_done = nullptr);
// Both GEMM launchers record `main_done` (if not null) on `stream` right
// after the main kernel, before the kernels that finish its output (the
// split fixup, the outlier scatter).
adahop_status record_main_done(hipEvent_t main_done, hipStream_t stream, const char* what);

}  // namespace adahop
