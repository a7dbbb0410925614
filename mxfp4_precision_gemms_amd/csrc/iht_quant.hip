// Zero + gather + IHT + MXFP4 quantization for gfx950.
//
// "AdaHOP ..." (arXiv 2604.02525), appendix kernel 2 (IHT and quantization)
// and kernel 1's last step (the chosen outlier lines are zeroed in the
// residual): the residual is rotated by a 1-D fast Walsh-Hadamard transform
// over blocks of 32 along the inner (contraction) dimension and quantized to
// MXFP4, one E8M0 scale per 32-element block (OCP MX v1.0 rule).
//
// HBM-bound: 2 bytes read and 0.53125 bytes written per element. Two
// directions:
//   contract COLS (blocks along a row, K contiguous in memory): one thread
//     owns 16 consecutive elements (two 16-byte loads); 2 lanes form a block.
//     Butterfly strides 1 to 8 run in registers, stride 16 across the 2 lanes
//     by a DPP lane swap; the block amax takes one more.
//   contract ROWS (blocks down a column): one thread owns 4 adjacent columns
//     of one 32-row block; each row is one 8-byte load; each column's
//     butterfly runs in registers; results are staged in LDS and written as
//     whole row segments.
// Extracted lines (the FOID indices) are found without searching: each
// workgroup reads the index list once, coalesced, before its tile, and marks
// the lines that fall inside its tile in LDS. The gathered lines are written
// line-major, [nz][length of a line].
// Both give bit-identical results to the same fp32 operations done one block
// at a time: each butterfly output is one rounded fp32 add or subtract, then
// one rounded multiply by fp32(1/sqrt(32)). The E2M1 codes come from gfx950's
// scaled FP4 convert (see pack8_e2m1).
#include <type_traits>

#include "quant_tiles.h"

#pragma clang fp contract(off)

namespace adahop {
namespace {

__global__ void __launch_bounds__(kRowThreads)
iht_quant_rowwise_kernel(const uint16_t* __restrict__ src, int64_t rows, int64_t K, int64_t ld,
                         int chunks_per_row, int hadamard, const int32_t* __restrict__ zidx,
                         int nz, int zaxis, uint8_t* __restrict__ codes,
                         uint8_t* __restrict__ scales, uint16_t* __restrict__ gathered,
                         int kchunk, int stream_src) {
  rowwise_tile(src, rows, K, ld, chunks_per_row, hadamard, zidx, nz, zaxis, codes, scales, gathered,
               kchunk, stream_src, blockIdx.x);
}

template <bool Vec, bool Had, bool NT>
__global__ void __launch_bounds__(kColThreads)
iht_quant_colwise_kernel(const uint16_t* __restrict__ src, int64_t K, int64_t outer, int64_t ld,
                         const int32_t* __restrict__ zidx, int nz, int zaxis,
                         uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                         uint16_t* __restrict__ gathered, int kchunk) {
  colwise_tile<Vec, Had, NT>(src, K, outer, ld, zidx, nz, zaxis, codes, scales, gathered, kchunk,
                             blockIdx.x, blockIdx.y);
}

// The quantization down the columns with the outer outlier product's
// partial sums formed in the same pass (colwise_oe_tiles): workgroup (x, y)
// takes column tile x and tile group y.
template <bool Vec, bool ByLine>
__global__ void __launch_bounds__(kColThreads, 2)
iht_quant_colwise_oe_kernel(const uint16_t* __restrict__ src, int64_t K, int64_t outer, int64_t ld,
                            uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int kchunk,
                            const uint16_t* __restrict__ lines, int k, int tiles_per_wg,
                            float* __restrict__ partials) {
  colwise_oe_tiles<Vec, ByLine>(src, K, outer, ld, codes, scales, kchunk, lines, k, tiles_per_wg,
                                partials, blockIdx.x, blockIdx.y);
}

}  // namespace

bool iht_quant_fits(int64_t rows, int64_t cols, int contract) {
  if (rows < 1 || cols < 1) return false;
  if (contract == ADAHOP_AXIS_COLS) {
    const int64_t cpr = (cols + kRowChunk - 1) / kRowChunk;
    return (rows + kRowRows - 1) / kRowRows * cpr <= 0x7FFFFFFFLL;
  }
  return (cols + kColOut - 1) / kColOut <= 0x7FFFFFFFLL &&
         (rows / 32 + kColBlocks - 1) / kColBlocks <= 65535;
}

adahop_status iht_quant_launch(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld,
                               int contract, int32_t hadamard_block, const int32_t* zero_idx,
                               int32_t nzero, int zero_axis, uint8_t* codes, uint8_t* scales,
                               uint16_t* gathered, int layout, hipStream_t stream,
                               bool stream_src) {
  const int kchunk = layout == ADAHOP_LAYOUT_KCHUNK ? 1 : 0;
  const int64_t Kc = contract == ADAHOP_AXIS_COLS ? cols : rows;
  if (kchunk && (Kc % 128 != 0 || (reinterpret_cast<uintptr_t>(scales) & 3u) != 0))
    return fail(ADAHOP_ERR_UNSUPPORTED, "iht_quant: K-chunked output needs K % 128 == 0");
  const int had = hadamard_block == 32 ? 1 : 0;
  if (contract == ADAHOP_AXIS_COLS) {
    const int64_t K = cols;
    const int64_t cpr = (K + kRowChunk - 1) / kRowChunk;
    const int64_t grid = (rows + kRowRows - 1) / kRowRows * cpr;
    if (grid > 0x7FFFFFFFLL) return fail(ADAHOP_ERR_UNSUPPORTED, "iht_quant: tensor too large");
    iht_quant_rowwise_kernel<<<dim3((unsigned)grid), dim3(kRowThreads), 0, stream>>>(
        src, rows, K, ld, (int)cpr, had, zero_idx, nzero, zero_axis, codes, scales, gathered,
        kchunk, stream_src ? 1 : 0);
  } else {
    const int64_t K = rows, outer = cols;
    const int64_t gx = (outer + kColOut - 1) / kColOut;
    const int64_t gy = (K / 32 + kColBlocks - 1) / kColBlocks;
    if (gx > 0x7FFFFFFFLL || gy > 65535)
      return fail(ADAHOP_ERR_UNSUPPORTED, "iht_quant: tensor too large");
    const dim3 grid((unsigned)gx, (unsigned)gy), block(kColThreads);
    // The per-row offsets of the vector path are 32-bit byte offsets from
    // the workgroup's first row: 512 rows of ld elements must stay below 2^31.
    const bool vec = ld % 4 == 0 && (reinterpret_cast<uintptr_t>(src) & 7u) == 0 &&
                     (int64_t)kColBlocks * 32 * ld * 2 < 0x7FFFFFFF;
    auto go = [&](auto V, auto H, auto N) {
      iht_quant_colwise_kernel<decltype(V)::value, decltype(H)::value, decltype(N)::value>
          <<<grid, block, 0, stream>>>(src, K, outer, ld, zero_idx, nzero, zero_axis, codes, scales,
                                       gathered, kchunk);
    };
    // The cache policy applies to the vector path's buffer loads only.
    if (vec && had && stream_src) go(std::true_type{}, std::true_type{}, std::true_type{});
    else if (vec && had) go(std::true_type{}, std::true_type{}, std::false_type{});
    else if (vec && stream_src) go(std::true_type{}, std::false_type{}, std::true_type{});
    else if (vec) go(std::true_type{}, std::false_type{}, std::false_type{});
    else if (had) go(std::false_type{}, std::true_type{}, std::false_type{});
    else go(std::false_type{}, std::false_type{}, std::false_type{});
  }
  return check_launch("iht_quant");
}

int iht_quant_oe_groups(int64_t K, int64_t outer, int32_t k, int* tiles_per_wg) {
  *tiles_per_wg = 0;
  if (k < 1 || k > kFusedOeMaxK || K < 32 || K % 32 != 0 || outer < 1) return 0;
  const int64_t ntiles = (K / 32 + kColBlocks - 1) / kColBlocks;
  const int64_t gx = (outer + kColOut - 1) / kColOut;
  // A workgroup takes enough tiles for about 512 workgroups in all (two per
  // CU), at least 4 (the partial sums then add at most half the operand's
  // bytes in traffic), at most 16.
  int64_t r = (ntiles * gx + 511) / 512;
  if (r < 4) r = 4;
  if (r > 16) r = 16;
  const int64_t groups = (ntiles + r - 1) / r;
  if (gx > 0x7FFFFFFFLL || groups > 65535) return 0;
  *tiles_per_wg = (int)r;
  return (int)groups;
}

adahop_status iht_quant_oe_launch(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld,
                                  uint8_t* codes, uint8_t* scales, int layout,
                                  const uint16_t* lines, int32_t k, int by_line, float* partials,
                                  hipStream_t stream) {
  const int64_t K = rows, outer = cols;
  int r = 0;
  const int groups = iht_quant_oe_groups(K, outer, k, &r);
  if (groups == 0) return fail(ADAHOP_ERR_UNSUPPORTED, "iht_quant: fused outlier product not applicable");
  const int kchunk = layout == ADAHOP_LAYOUT_KCHUNK ? 1 : 0;
  if (kchunk && (K % 128 != 0 || (reinterpret_cast<uintptr_t>(scales) & 3u) != 0))
    return fail(ADAHOP_ERR_UNSUPPORTED, "iht_quant: K-chunked output needs K % 128 == 0");
  if ((reinterpret_cast<uintptr_t>(lines) & 15u) != 0)
    return fail(ADAHOP_ERR_UNSUPPORTED, "iht_quant: lines must be 16-byte aligned");
  const dim3 grid((unsigned)((outer + kColOut - 1) / kColOut), (unsigned)groups), block(kColThreads);
  const bool vec = ld % 4 == 0 && (reinterpret_cast<uintptr_t>(src) & 7u) == 0 &&
                   (int64_t)kColBlocks * 32 * ld * 2 < 0x7FFFFFFF;
  auto go = [&](auto V, auto L) {
    iht_quant_colwise_oe_kernel<decltype(V)::value, decltype(L)::value><<<grid, block, 0, stream>>>(
        src, K, outer, ld, codes, scales, kchunk, lines, k, r, partials);
  };
  if (vec && by_line) go(std::true_type{}, std::true_type{});
  else if (vec) go(std::true_type{}, std::false_type{});
  else if (by_line) go(std::false_type{}, std::true_type{});
  else go(std::false_type{}, std::false_type{});
  return check_launch("iht_quant_oe");
}

}  // namespace adahop
