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
//     owns 8 consecutive elements (a 16-byte load); 4 lanes form a block.
//     Butterfly strides 1, 2, 4 run in registers, strides 8 and 16 across the
//     4 lanes by lane shuffles; the block amax takes two shuffles.
//   contract ROWS (blocks down a column): one thread owns one column block of
//     32 rows; consecutive lanes read consecutive columns, so each row read of
//     a wave is one contiguous segment; the whole butterfly runs in registers.
// Both give bit-identical results to the same fp32 operations done one block
// at a time: each butterfly output is one rounded fp32 add or subtract, then
// one rounded multiply by fp32(1/sqrt(32)).
#include "adahop_internal.h"

#pragma clang fp contract(off)

namespace adahop {
namespace {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// E2M1 magnitude (0..7) of v >= 0: the nearest of {0,.5,1,1.5,2,3,4,6},
// ties to the even code, saturating. Each comparison passes one midpoint;
// at a midpoint the comparison is <= or < so that the even code wins.
__device__ __forceinline__ uint32_t e2m1_magnitude(float v) {
  return (uint32_t)(v > 0.25f) + (uint32_t)(v >= 0.75f) + (uint32_t)(v > 1.25f) +
         (uint32_t)(v >= 1.75f) + (uint32_t)(v > 2.5f) + (uint32_t)(v >= 3.5f) +
         (uint32_t)(v > 5.0f);
}

// Shared exponent s = floor(log2 amax) - 2, clamped below at -127 (this also
// covers amax = 0 and subnormal amax, whose byte is 0x00). amax is finite.
__device__ __forceinline__ int block_exponent(float amax) {
  int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  int s = e - 127 - 2;
  return s < -127 ? -127 : s;
}

// 2^-s as an fp32 for s in [-127, 125] (a normal number).
__device__ __forceinline__ float inv_pow2(int s) {
  return __uint_as_float((uint32_t)(127 - s) << 23);
}

__device__ __forceinline__ uint32_t e2m1_code(float y, float inv_scale) {
  uint32_t sign = __float_as_uint(y) >> 31;
  return (sign << 3) | e2m1_magnitude(fabsf(y) * inv_scale);
}

// Position of v in the ascending list idx[0..n), or -1.
__device__ __forceinline__ int find_sorted(const int32_t* idx, int n, int64_t v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)idx[mid] < v) lo = mid + 1; else hi = mid;
  }
  return (lo < n && (int64_t)idx[lo] == v) ? lo : -1;
}

// First position with idx[pos] >= v.
__device__ __forceinline__ int lower_bound(const int32_t* idx, int n, int64_t v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)idx[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

constexpr int kRowThreads = 256;
constexpr int kRowChunk = kRowThreads * 8;   // elements of one row per workgroup

// contract COLS: src [rows][K], K contiguous. Grid: rows * ceil(K / kRowChunk).
__global__ void __launch_bounds__(kRowThreads)
iht_quant_rowwise_kernel(const uint16_t* __restrict__ src, int64_t K, int64_t ld,
                         int chunks_per_row, int hadamard, const int32_t* __restrict__ zidx,
                         int nz, int zaxis, uint8_t* __restrict__ codes,
                         uint8_t* __restrict__ scales, uint16_t* __restrict__ gathered) {
  const int64_t r = blockIdx.x / chunks_per_row;
  const int64_t col0 = (int64_t)(blockIdx.x % chunks_per_row) * kRowChunk + threadIdx.x * 8;
  const bool active = col0 < K;   // K % 32 == 0: whole 4-lane groups agree
  const int lane4 = threadIdx.x & 3;

  uint4 raw = make_uint4(0, 0, 0, 0);
  if (active) raw = *reinterpret_cast<const uint4*>(src + r * ld + col0);
  uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
    y[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }

  if (nz > 0 && active) {
    if (zaxis == ADAHOP_AXIS_ROWS) {
      int p = find_sorted(zidx, nz, r);
      if (p >= 0) {
        if (gathered) *reinterpret_cast<uint4*>(gathered + (int64_t)p * K + col0) = raw;
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = 0.0f;
      }
    } else {
      // Registers are indexed by unrolled constants only: collect a mask of
      // the zeroed positions, then select.
      uint32_t zmask = 0;
      for (int p = lower_bound(zidx, nz, col0); p < nz && zidx[p] < col0 + 8; ++p) {
        const int i = (int)(zidx[p] - col0);
        zmask |= 1u << i;
        if (gathered) {
          const int wi = i >> 1;
          const uint32_t word = wi == 0 ? w[0] : wi == 1 ? w[1] : wi == 2 ? w[2] : w[3];
          gathered[r * nz + p] = (uint16_t)((word >> (16 * (i & 1))) & 0xFFFFu);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = ((zmask >> i) & 1u) ? 0.0f : y[i];
    }
  }

  if (hadamard) {
    // strides 1, 2, 4 inside the lane
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i & h) continue;
        float a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
    }
    // stride 8: lanes (0,1) and (2,3) of the group; stride 16: lanes (0,2) and (1,3)
#pragma unroll
    for (int step = 1; step <= 2; step <<= 1) {
      const bool upper = (lane4 & step) != 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float o = __shfl_xor(y[i], step);
        y[i] = upper ? (o - y[i]) : (y[i] + o);
      }
    }
    const float c = __uint_as_float(0x3E3504F3u);   // fp32(1/sqrt(32))
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = y[i] * c;
  }

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int s = block_exponent(amax);
  const float inv = inv_pow2(s);
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) packed |= e2m1_code(y[i], inv) << (4 * i);
  if (active) {
    *reinterpret_cast<uint32_t*>(codes + r * (K / 2) + col0 / 2) = packed;
    if (lane4 == 0) scales[r * (K / 32) + col0 / 32] = (uint8_t)(s + 127);
  }
}

constexpr int kColLanes = 64;    // columns per workgroup
constexpr int kColBlocks = 4;    // 32-row blocks per workgroup

// contract ROWS: src [K][outer], blocks run down columns. Grid:
// (ceil(outer / 64), ceil(K / 32 / 4)); thread (x, y) owns column
// blockIdx.x*64 + x and block blockIdx.y*4 + y.
__global__ void __launch_bounds__(kColLanes * kColBlocks)
iht_quant_colwise_kernel(const uint16_t* __restrict__ src, int64_t K, int64_t outer, int64_t ld,
                         int hadamard, const int32_t* __restrict__ zidx, int nz, int zaxis,
                         uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                         uint16_t* __restrict__ gathered) {
  const int64_t c = (int64_t)blockIdx.x * kColLanes + threadIdx.x;
  const int64_t b = (int64_t)blockIdx.y * kColBlocks + threadIdx.y;
  if (c >= outer || b * 32 >= K) return;
  const int64_t t0 = b * 32;

  float y[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) y[j] = bf16_bits_to_f32(src[(t0 + j) * ld + c]);

  if (nz > 0) {
    if (zaxis == ADAHOP_AXIS_COLS) {
      int p = find_sorted(zidx, nz, c);
      if (p >= 0) {
        if (gathered)
          for (int j = 0; j < 32; ++j) gathered[(t0 + j) * nz + p] = src[(t0 + j) * ld + c];
#pragma unroll
        for (int j = 0; j < 32; ++j) y[j] = 0.0f;
      }
    } else {
      for (int p = lower_bound(zidx, nz, t0); p < nz && zidx[p] < t0 + 32; ++p) {
        int j = (int)(zidx[p] - t0);
        if (gathered) gathered[(int64_t)p * outer + c] = src[(t0 + j) * ld + c];
        // y[j] = 0 with a runtime j: select over the unrolled block
#pragma unroll
        for (int q = 0; q < 32; ++q) y[q] = (q == j) ? 0.0f : y[q];
      }
    }
  }

  if (hadamard) {
#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i & h) continue;
        float a = y[i], bb = y[i + h];
        y[i] = a + bb;
        y[i + h] = a - bb;
      }
    }
    const float cst = __uint_as_float(0x3E3504F3u);   // fp32(1/sqrt(32))
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = y[i] * cst;
  }

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(y[i]));
  const int s = block_exponent(amax);
  const float inv = inv_pow2(s);
  uint32_t q[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 32; ++i) q[i >> 3] |= e2m1_code(y[i], inv) << (4 * (i & 7));
  *reinterpret_cast<uint4*>(codes + c * (K / 2) + b * 16) = make_uint4(q[0], q[1], q[2], q[3]);
  scales[c * (K / 32) + b] = (uint8_t)(s + 127);
}

}  // namespace

adahop_status iht_quant_launch(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld,
                               int contract, int32_t hadamard_block, const int32_t* zero_idx,
                               int32_t nzero, int zero_axis, uint8_t* codes, uint8_t* scales,
                               uint16_t* gathered, hipStream_t stream) {
  const int had = hadamard_block == 32 ? 1 : 0;
  if (contract == ADAHOP_AXIS_COLS) {
    const int64_t K = cols;
    const int64_t cpr = (K + kRowChunk - 1) / kRowChunk;
    const int64_t grid = rows * cpr;
    if (grid > 0x7FFFFFFFLL) return fail(ADAHOP_ERR_UNSUPPORTED, "iht_quant: tensor too large");
    iht_quant_rowwise_kernel<<<dim3((unsigned)grid), dim3(kRowThreads), 0, stream>>>(
        src, K, ld, (int)cpr, had, zero_idx, nzero, zero_axis, codes, scales, gathered);
  } else {
    const int64_t K = rows, outer = cols;
    const int64_t gx = (outer + kColLanes - 1) / kColLanes;
    const int64_t gy = (K / 32 + kColBlocks - 1) / kColBlocks;
    if (gx > 0x7FFFFFFFLL || gy > 65535)
      return fail(ADAHOP_ERR_UNSUPPORTED, "iht_quant: tensor too large");
    iht_quant_colwise_kernel<<<dim3((unsigned)gx, (unsigned)gy), dim3(kColLanes, kColBlocks), 0,
                               stream>>>(src, K, outer, ld, had, zero_idx, nzero, zero_axis,
                                         codes, scales, gathered);
  }
  return check_launch("iht_quant");
}

}  // namespace adahop
