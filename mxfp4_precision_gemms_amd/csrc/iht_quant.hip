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
//     by a lane shuffle; the block amax takes one shuffle.
//   contract ROWS (blocks down a column): one thread owns 4 adjacent columns
//     of one 32-row block; each row is one 8-byte load, so a wave's row read
//     is 512 contiguous bytes; each column's butterfly runs in registers.
// Both give bit-identical results to the same fp32 operations done one block
// at a time: each butterfly output is one rounded fp32 add or subtract, then
// one rounded multiply by fp32(1/sqrt(32)). The E2M1 codes come from gfx950's
// scaled FP4 convert (see pack8_e2m1).
#include "adahop_internal.h"

#pragma clang fp contract(off)

namespace adahop {
namespace {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Shared exponent s = floor(log2 amax) - 2, clamped below at -127 (this also
// covers amax = 0 and subnormal amax, whose byte is 0x00). amax is finite.
__device__ __forceinline__ int block_exponent(float amax) {
  int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  int s = e - 127 - 2;
  return s < -127 ? -127 : s;
}

// E2M1 codes of y[0..7] / 2^s, packed 8 per dword (element 2j in the low
// nibble of byte j). v_cvt_scalef32_pk_fp4_f32 takes the scale as an fp32
// whose exponent field is the E8M0 byte s + 127, divides, rounds to nearest
// (ties to the even code), saturates at 6 and keeps the sign bit -- the OCP
// MX conversion, checked bit-exact against the scalar rule over every finite
// bf16 value at scale exponents from -127 to 125.
__device__ __forceinline__ uint32_t pack8_e2m1(const float* y, float scale) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], scale, 3);
  return w;
}

__device__ __forceinline__ float e8m0_as_f32(int s) {
  return __uint_as_float((uint32_t)(s + 127) << 23);
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
constexpr int kRowChunk = kRowThreads * 16;  // elements of one row per workgroup

// contract COLS: src [rows][K], K contiguous. Grid: rows * ceil(K / kRowChunk).
// A lane owns 16 consecutive elements (two 16-byte loads), two lanes form a
// 32-block: butterfly strides 1..8 in registers, stride 16 by one shuffle.
__global__ void __launch_bounds__(kRowThreads)
iht_quant_rowwise_kernel(const uint16_t* __restrict__ src, int64_t K, int64_t ld,
                         int chunks_per_row, int hadamard, const int32_t* __restrict__ zidx,
                         int nz, int zaxis, uint8_t* __restrict__ codes,
                         uint8_t* __restrict__ scales, uint16_t* __restrict__ gathered) {
  const int64_t r = blockIdx.x / chunks_per_row;
  const int64_t col0 = (int64_t)(blockIdx.x % chunks_per_row) * kRowChunk + threadIdx.x * 16;
  const bool active = col0 < K;   // K % 32 == 0: both lanes of a block agree
  const bool upper = (threadIdx.x & 1) != 0;

  uint4 raw0 = make_uint4(0, 0, 0, 0), raw1 = make_uint4(0, 0, 0, 0);
  if (active) {
    raw0 = *reinterpret_cast<const uint4*>(src + r * ld + col0);
    raw1 = *reinterpret_cast<const uint4*>(src + r * ld + col0 + 8);
  }
  const uint32_t w[8] = {raw0.x, raw0.y, raw0.z, raw0.w, raw1.x, raw1.y, raw1.z, raw1.w};
  float y[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    y[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
    y[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }

  if (nz > 0 && active) {
    if (zaxis == ADAHOP_AXIS_ROWS) {
      const int p = find_sorted(zidx, nz, r);
      if (p >= 0) {
        if (gathered) {
          *reinterpret_cast<uint4*>(gathered + (int64_t)p * K + col0) = raw0;
          *reinterpret_cast<uint4*>(gathered + (int64_t)p * K + col0 + 8) = raw1;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = 0.0f;
      }
    } else {
      // Registers are indexed by unrolled constants only: collect a mask of
      // the zeroed positions, then select.
      uint32_t zmask = 0;
      for (int p = lower_bound(zidx, nz, col0); p < nz && zidx[p] < col0 + 16; ++p) {
        const int i = (int)(zidx[p] - col0);
        zmask |= 1u << i;
        if (gathered) {
          uint32_t word = 0;
#pragma unroll
          for (int q = 0; q < 8; ++q) word = (q == (i >> 1)) ? w[q] : word;
          gathered[r * nz + p] = (uint16_t)((word >> (16 * (i & 1))) & 0xFFFFu);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = ((zmask >> i) & 1u) ? 0.0f : y[i];
    }
  }

  if (hadamard) {
    // strides 1, 2, 4, 8 inside the lane
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i & h) continue;
        const float a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
    }
    // stride 16: the two lanes of the block
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float o = __shfl_xor(y[i], 1);
      y[i] = upper ? (o - y[i]) : (y[i] + o);
    }
    const float c = __uint_as_float(0x3E3504F3u);   // fp32(1/sqrt(32))
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = y[i] * c;
  }

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(y[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  const int sx = block_exponent(amax);
  const float scale = e8m0_as_f32(sx);
  const uint32_t lo = pack8_e2m1(y, scale), hi = pack8_e2m1(y + 8, scale);
  if (active) {
    *reinterpret_cast<uint2*>(codes + r * (K / 2) + col0 / 2) = make_uint2(lo, hi);
    if (!upper) scales[r * (K / 32) + col0 / 32] = (uint8_t)(sx + 127);
  }
}

constexpr int kColLanes = 64;    // columns per workgroup
constexpr int kColBlocks = 4;    // 32-row blocks per workgroup

// contract ROWS, 4 columns per thread: thread (x, y) of a 64 x 4 workgroup
// owns columns 4 (64 blockIdx.x + x) .. +3 of block blockIdx.y * 4 + y. Each
// row of the block is one 8-byte load (a wave reads 512 contiguous bytes);
// the columns are then rotated and quantized one after another from
// registers. Vec: the rows allow aligned 8-byte loads (ld % 4 == 0, base
// 8-byte aligned); otherwise the loads are per element.
template <bool Vec>
__global__ void __launch_bounds__(kColLanes * kColBlocks)
iht_quant_colwise4_kernel(const uint16_t* __restrict__ src, int64_t K, int64_t outer, int64_t ld,
                          int hadamard, const int32_t* __restrict__ zidx, int nz, int zaxis,
                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                          uint16_t* __restrict__ gathered) {
  const int64_t c0 = ((int64_t)blockIdx.x * kColLanes + threadIdx.x) * 4;
  const int64_t b = (int64_t)blockIdx.y * kColBlocks + threadIdx.y;
  if (c0 >= outer || b * 32 >= K) return;
  const int64_t t0 = b * 32;
  const bool whole = Vec && c0 + 4 <= outer;

  uint32_t w[32][2];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    if (whole) {
      const uint2 q = *reinterpret_cast<const uint2*>(src + (t0 + j) * ld + c0);
      w[j][0] = q.x;
      w[j][1] = q.y;
    } else {
      uint32_t h[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) h[q] = c0 + q < outer ? src[(t0 + j) * ld + c0 + q] : 0u;
      w[j][0] = h[0] | (h[1] << 16);
      w[j][1] = h[2] | (h[3] << 16);
    }
  }

  // Rows of this block that are extracted lines (zero_axis ROWS).
  uint32_t rmask = 0;
  if (nz > 0 && zaxis == ADAHOP_AXIS_ROWS) {
    for (int p = lower_bound(zidx, nz, t0); p < nz && zidx[p] < t0 + 32; ++p) {
      const int j = (int)(zidx[p] - t0);
      rmask |= 1u << j;
      if (gathered) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (c0 + q < outer) gathered[(int64_t)p * outer + c0 + q] = src[(t0 + j) * ld + c0 + q];
      }
    }
  }

#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t c = c0 + q;
    if (c >= outer) break;
    float y[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t h = (w[j][q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
      y[j] = ((rmask >> j) & 1u) ? 0.0f : bf16_bits_to_f32(h);
    }
    if (nz > 0 && zaxis == ADAHOP_AXIS_COLS) {
      const int p = find_sorted(zidx, nz, c);
      if (p >= 0) {
        if (gathered) {
#pragma unroll
          for (int j = 0; j < 32; ++j)
            gathered[(t0 + j) * nz + p] = (uint16_t)((w[j][q >> 1] >> (16 * (q & 1))) & 0xFFFFu);
        }
#pragma unroll
        for (int j = 0; j < 32; ++j) y[j] = 0.0f;
      }
    }
    if (hadamard) {
#pragma unroll
      for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          if (i & h) continue;
          const float a = y[i], bb = y[i + h];
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
    const int sx = block_exponent(amax);
    const float scale = e8m0_as_f32(sx);
    *reinterpret_cast<uint4*>(codes + c * (K / 2) + b * 16) =
        make_uint4(pack8_e2m1(y, scale), pack8_e2m1(y + 8, scale), pack8_e2m1(y + 16, scale),
                   pack8_e2m1(y + 24, scale));
    scales[c * (K / 32) + b] = (uint8_t)(sx + 127);
  }
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
    const int64_t gx = (outer + 4 * kColLanes - 1) / (4 * kColLanes);
    const int64_t gy = (K / 32 + kColBlocks - 1) / kColBlocks;
    if (gx > 0x7FFFFFFFLL || gy > 65535)
      return fail(ADAHOP_ERR_UNSUPPORTED, "iht_quant: tensor too large");
    const bool vec = ld % 4 == 0 && (reinterpret_cast<uintptr_t>(src) & 7u) == 0;
    const dim3 grid((unsigned)gx, (unsigned)gy), block(kColLanes, kColBlocks);
    if (vec)
      iht_quant_colwise4_kernel<true><<<grid, block, 0, stream>>>(
          src, K, outer, ld, had, zero_idx, nzero, zero_axis, codes, scales, gathered);
    else
      iht_quant_colwise4_kernel<false><<<grid, block, 0, stream>>>(
          src, K, outer, ld, had, zero_idx, nzero, zero_axis, codes, scales, gathered);
  }
  return check_launch("iht_quant");
}

}  // namespace adahop
