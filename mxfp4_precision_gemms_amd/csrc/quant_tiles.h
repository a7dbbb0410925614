// Zero + gather + IHT + MXFP4 tiles as device code (appendix kernel 2 of
// "AdaHOP ..." (arXiv 2604.02525)), included by iht_quant.hip (the
// quantization kernels) and foid.hip (a quantization beside FOID's selection
// in one launch). How the tiles work is described in iht_quant.hip.
#pragma once

#include "adahop_internal.h"

#pragma clang fp contract(off)

namespace adahop {
namespace {

// Cache-policy immediate of a buffer load: NT (non-temporal, streaming).
constexpr int kLoadNT = 2;
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

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

// The value held by lane l ^ 1 (DPP quad permutation [1, 0, 3, 2]: a VALU
// operand modifier, no LDS traffic).
__device__ __forceinline__ float pair_swap(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}

__device__ __forceinline__ float e8m0_as_f32(int s) {
  return __uint_as_float((uint32_t)(s + 127) << 23);
}

constexpr int kRowThreads = 256;
constexpr int kRowRows = kRowThreads / 64;   // rows per workgroup, one wave each
constexpr int kRowChunk = 64 * 16;           // columns per workgroup

// contract COLS: src [rows][K], K contiguous. A workgroup takes 4 rows x 1024
// columns, one wave per row. A lane owns 16 consecutive elements (two 16-byte
// loads), two lanes form a 32-block: butterfly strides 1..8 in registers,
// stride 16 by one shuffle. Row-major output goes out from registers (a
// wave's 512 code bytes are contiguous); K-chunked output is staged in LDS
// and written as runs of 4 rows x 64 bytes, whole lines.
// `bx`: this workgroup's tile (the kernel's block index).
__device__ __forceinline__ void rowwise_tile(const uint16_t* __restrict__ src, int64_t rows, int64_t K,
                                             int64_t ld, int chunks_per_row, int hadamard,
                                             const int32_t* __restrict__ zidx, int nz, int zaxis,
                                             uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                             uint16_t* __restrict__ gathered, int kchunk, int stream_src,
                                             int64_t bx) {
  // Extracted lines inside this tile: each row's position in the index list
  // (zero_axis ROWS, -1 if none), or a mask of the columns (zero_axis COLS).
  __shared__ int32_t s_rowpos[kRowRows];
  __shared__ uint32_t s_cmask[kRowChunk / 32];
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[kRowRows][kRowChunk / 2];
  __shared__ __attribute__((aligned(16))) uint8_t s_scales[kRowRows][kRowChunk / 32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r0 = bx / chunks_per_row * kRowRows;
  const int64_t r = r0 + wave;
  const int64_t cbase = bx % chunks_per_row * kRowChunk;
  const int64_t col0 = cbase + lane * 16;
  const bool active = r < rows && col0 < K;   // K % 32 == 0: both lanes of a block agree
  const bool upper = (lane & 1) != 0;

  // This thread's share of the index list, loaded before the rows so that
  // waiting for it does not wait for the rows.
  int zv[kMaxK / kRowThreads];
#pragma unroll
  for (int q = 0; q < kMaxK / kRowThreads; ++q) {
    const int i = tid + q * kRowThreads;
    zv[q] = i < nz ? zidx[i] : -1;
  }
  uint4 raw0 = make_uint4(0, 0, 0, 0), raw1 = make_uint4(0, 0, 0, 0);
  if (active) {
    // Read once: non-temporal loads, as in the column-direction kernel
    // (ordinary ones when another kernel reads the source again soon).
    const v4u32* p = reinterpret_cast<const v4u32*>(src + r * ld + col0);
    v4u32 a, b;
    if (stream_src) {
      a = __builtin_nontemporal_load(p);
      b = __builtin_nontemporal_load(p + 1);
    } else {
      a = p[0];
      b = p[1];
    }
    raw0 = make_uint4(a.x, a.y, a.z, a.w);
    raw1 = make_uint4(b.x, b.y, b.z, b.w);
  }

  if (tid < kRowRows) s_rowpos[tid] = -1;
  if (tid < kRowChunk / 32) s_cmask[tid] = 0;
  __syncthreads();
  if (nz > 0) {
#pragma unroll
    for (int q = 0; q < kMaxK / kRowThreads; ++q) {
      if (zv[q] < 0) continue;
      const int i = tid + q * kRowThreads;
      if (zaxis == ADAHOP_AXIS_ROWS) {
        if (zv[q] >= r0 && zv[q] < r0 + kRowRows && zv[q] < rows) s_rowpos[zv[q] - r0] = i;
      } else {
        const int64_t d = (int64_t)zv[q] - cbase;
        if (d >= 0 && d < kRowChunk && zv[q] < K) {
          atomicOr(&s_cmask[d / 32], 1u << (d % 32));
          // An extracted column: gathered [nz][rows], elements (i, r0 .. r0 + 3).
          if (gathered) {
            for (int j = 0; j < kRowRows; ++j)
              if (r0 + j < rows) gathered[(int64_t)i * rows + r0 + j] = src[(r0 + j) * ld + zv[q]];
          }
        }
      }
    }
  }
  __syncthreads();

  const uint32_t w[8] = {raw0.x, raw0.y, raw0.z, raw0.w, raw1.x, raw1.y, raw1.z, raw1.w};
  float y[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    y[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
    y[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
  if (nz > 0 && active) {
    if (zaxis == ADAHOP_AXIS_ROWS) {
      const int p = s_rowpos[wave];
      if (p >= 0) {
        if (gathered) {
          *reinterpret_cast<uint4*>(gathered + (int64_t)p * K + col0) = raw0;
          *reinterpret_cast<uint4*>(gathered + (int64_t)p * K + col0 + 8) = raw1;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = 0.0f;
      }
    } else {
      // lane * 16 is a multiple of 16: this lane's 16 columns sit in one word.
      const int d = lane * 16;
      const uint32_t zmask = (s_cmask[d / 32] >> (d % 32)) & 0xFFFFu;
      if (zmask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = ((zmask >> i) & 1u) ? 0.0f : y[i];
      }
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
    // stride 16: the two lanes of the block. The lower lane forms y + o, the
    // upper one o - y, both as o + (+-y): negation is exact and addition
    // commutes, so the sums are the same bits.
    const uint32_t neg = upper ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float o = pair_swap(y[i]);
      y[i] = o + __uint_as_float(__float_as_uint(y[i]) ^ neg);
    }
    const float c = __uint_as_float(0x3E3504F3u);   // fp32(1/sqrt(32))
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = y[i] * c;
  }

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(y[i]));
  amax = fmaxf(amax, pair_swap(amax));
  const int sx = block_exponent(amax);
  const float scale = e8m0_as_f32(sx);
  const uint32_t lo = pack8_e2m1(y, scale), hi = pack8_e2m1(y + 8, scale);
  if (!kchunk) {
    if (active) {
      *reinterpret_cast<uint2*>(codes + r * (K / 2) + col0 / 2) = make_uint2(lo, hi);
      if (!upper) scales[r * (K / 32) + col0 / 32] = (uint8_t)(sx + 127);
    }
    return;
  }
  // [K/128][rows][64] and [K/128][rows][4]: chunk q of this tile is rows
  // r0 .. r0 + 3 x 64 bytes, one contiguous run (K % 128 == 0).
  *reinterpret_cast<uint2*>(&s_codes[wave][lane * 8]) = make_uint2(lo, hi);
  // Scale bytes of a 128-long chunk go in the order 0, 2, 1, 3 (the layout
  // the GEMM reads 16 bits at a time per half-wave).
  if (!upper) {
    const int b = lane / 2;              // block within the workgroup's row
    s_scales[wave][(b & ~3) | ((b & 1) << 1) | ((b >> 1) & 1)] = (uint8_t)(sx + 127);
  }
  __syncthreads();
  const int nrow = (int)(rows - r0 < kRowRows ? rows - r0 : kRowRows);
  const int nch = (int)((K - cbase) / 128 < kRowChunk / 128 ? (K - cbase) / 128 : kRowChunk / 128);
  const int64_t c0 = cbase / 128;
  if (tid < (kRowChunk / 128) * kRowRows * 4) {
    const int q = tid / (kRowRows * 4), piece = tid % (kRowRows * 4);
    const int row = piece / 4, part = piece % 4;
    if (q < nch && row < nrow)
      *reinterpret_cast<uint4*>(codes + ((c0 + q) * rows + r0) * 64 + piece * 16) =
          *reinterpret_cast<const uint4*>(&s_codes[row][q * 64 + part * 16]);
  }
  if (tid < (kRowChunk / 128) * kRowRows) {
    const int q = tid / kRowRows, row = tid % kRowRows;
    if (q < nch && row < nrow)
      *reinterpret_cast<uint32_t*>(scales + ((c0 + q) * rows + r0 + row) * 4) =
          *reinterpret_cast<const uint32_t*>(&s_scales[row][q * 4]);
  }
}

// contract ROWS: a 256-thread workgroup owns 256 output rows (columns of the
// source) x 4 blocks of 32 contraction positions, one block per wave. Thread
// t takes the 4 adjacent columns 4 (t % 64) .. +3 of block t / 64: each of
// the block's 32 rows is one 8-byte load (a wave reads 512 contiguous bytes
// of a row), and the columns are rotated and quantized one after another
// from registers. Codes and scales go to LDS first, then out as whole
// segments: K-chunked, the tile's 128 contraction positions are one chunk,
// 256 rows x 64 bytes contiguous; row-major, 64 code bytes and 4 scale bytes
// per output row. Vec: the rows allow aligned 8-byte loads (ld % 4 == 0,
// base 8-byte aligned); otherwise loads are per element.
constexpr int kColThreads = 256;
constexpr int kColGroups = 64;                 // 4-column groups per workgroup
constexpr int kColOut = 4 * kColGroups;        // output rows per workgroup
constexpr int kColBlocks = kColThreads / kColGroups;   // 32-row blocks per workgroup
constexpr int kColPitch = kColBlocks * 16 + 16;        // LDS bytes per output row (padded)

// Loads the 32 x 4 bf16 block of one thread: rows t0 .. t0 + 31 (t0 =
// 32 (bbase + bi)) of columns c0 .. c0 + 3, row j packed in w[j] (columns
// c0, c0 + 1 in w[j][0]). Columns past `outer` read as +0.
template <bool Vec, bool NT>
__device__ __forceinline__ void colwise_load(uint32_t (&w)[32][2], const uint16_t* __restrict__ src,
                                             int64_t ld, int64_t outer, int64_t bbase, int bi,
                                             int64_t c0) {
  const int64_t t0 = (bbase + bi) * 32;
  if (Vec && c0 + 4 <= outer) {
    // Row j of the block is at byte j * ld * 2 from the block's first row:
    // a scalar offset, so the 32 loads need no per-lane address arithmetic.
    // The source is read once: non-temporal loads (cache policy NT) stream
    // it past the caches (7.3 against 6.6 TB/s for this load pattern alone,
    // measured) and leave them to the packed output the GEMM reads next;
    // ordinary loads (NT false) when another kernel reads the source again
    // soon after.
    const uint16_t* blk = src + (bbase * 32) * ld;     // workgroup-uniform
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(blk), 0, 0x7FFFFFFF, 0x00020000);
    const int voff = (int)((bi * 32 * ld + c0) * 2);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const auto q = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, (int)(j * ld * 2), NT ? kLoadNT : 0);
      w[j][0] = q[0];
      w[j][1] = q[1];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      uint32_t h[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) h[q] = c0 + q < outer ? src[(t0 + j) * ld + c0 + q] : 0u;
      w[j][0] = h[0] | (h[1] << 16);
      w[j][1] = h[2] | (h[3] << 16);
    }
  }
}

// Rotates and quantizes the thread's 4 columns (tile columns 4 cg .. + 3)
// of block bi one after another from registers; codes and scale bytes go to
// the tile's LDS rows.
template <bool Had>
__device__ __forceinline__ void colwise_quant_to_lds(const uint32_t (&w)[32][2], int64_t c0,
                                                     int64_t outer, int cg, int bi,
                                                     uint8_t* s_codes, uint8_t* s_scales) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t c = c0 + q;
    if (c >= outer) continue;
    float y[32];
    // bf16 -> fp32: the low half shifted up, or the high half masked.
#pragma unroll
    for (int j = 0; j < 32; ++j)
      y[j] = __uint_as_float((q & 1) ? (w[j][q >> 1] & 0xFFFF0000u) : (w[j][q >> 1] << 16));
    if (Had) {
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
    const int r = 4 * cg + q;
    *reinterpret_cast<uint4*>(&s_codes[r * kColPitch + bi * 16]) =
        make_uint4(pack8_e2m1(y, scale), pack8_e2m1(y + 8, scale), pack8_e2m1(y + 16, scale),
                   pack8_e2m1(y + 24, scale));
    s_scales[r * kColBlocks + bi] = (uint8_t)(sx + 127);
  }
}

// Write-out of a tile from LDS: output row r of the tile gets its blocks
// bbase .. bbase + nb - 1.
__device__ __forceinline__ void colwise_write_tile(const uint8_t* s_codes, const uint8_t* s_scales,
                                                   uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales, int kchunk,
                                                   int64_t K, int64_t outer, int64_t cbase,
                                                   int64_t bbase) {
  const int tid = threadIdx.x;
  const int64_t nblocks = K / 32;
  const int nrow = (int)(outer - cbase < kColOut ? outer - cbase : kColOut);
  const int nb = (int)(nblocks - bbase < kColBlocks ? nblocks - bbase : kColBlocks);
  if (kchunk) {
    // [K/128][outer][64] and [K/128][outer][4]: chunk q of this tile (4
    // blocks) is 64 consecutive rows x 64 bytes, one contiguous run
    // (K % 128 == 0, so nb is a multiple of 4).
    const int64_t c0k = bbase / 4;
    for (int i = tid; i < kColOut * kColBlocks; i += kColThreads) {
      const int q = i / (kColOut * 4), r = (i / 4) % kColOut, piece = i % 4;
      if (r < nrow && 4 * q < nb)
        *reinterpret_cast<uint4*>(codes + ((c0k + q) * outer + cbase + r) * 64 + piece * 16) =
            *reinterpret_cast<const uint4*>(&s_codes[r * kColPitch + (4 * q + piece) * 16]);
    }
    {
      const int q = tid / kColOut, r = tid % kColOut;
      if (r < nrow && 4 * q < nb)
      {
        // block scales 0, 1, 2, 3 of the chunk stored in the order 0, 2, 1, 3
        const uint32_t v = *reinterpret_cast<const uint32_t*>(&s_scales[r * kColBlocks + 4 * q]);
        *reinterpret_cast<uint32_t*>(scales + ((c0k + q) * outer + cbase + r) * 4) =
            (v & 0xFF0000FFu) | ((v >> 8) & 0xFF00u) | ((v << 8) & 0xFF0000u);
      }
    }
    return;
  }
  for (int i = tid; i < kColOut * kColBlocks; i += kColThreads) {
    const int r = i / kColBlocks, ch = i % kColBlocks;
    if (r < nrow && ch < nb)
      *reinterpret_cast<uint4*>(codes + (cbase + r) * (K / 2) + (bbase + ch) * 16) =
          *reinterpret_cast<const uint4*>(&s_codes[r * kColPitch + ch * 16]);
  }
  const bool vec_scales = nb == kColBlocks && nblocks % kColBlocks == 0 &&
                          (reinterpret_cast<uintptr_t>(scales) & (kColBlocks - 1)) == 0;
  if (vec_scales) {
    if (tid < nrow)
      *reinterpret_cast<uint32_t*>(scales + (cbase + tid) * nblocks + bbase) =
          *reinterpret_cast<const uint32_t*>(&s_scales[tid * kColBlocks]);
  } else {
    for (int i = tid; i < kColOut * kColBlocks; i += kColThreads) {
      const int r = i / kColBlocks, ch = i % kColBlocks;
      if (r < nrow && ch < nb) scales[(cbase + r) * nblocks + bbase + ch] = s_scales[r * kColBlocks + ch];
    }
  }
}

// `bx`, `by`: this workgroup's tile of columns and of 32-row blocks (the
// kernel's block indices).
template <bool Vec, bool Had, bool NT>
__device__ __forceinline__ void colwise_tile(const uint16_t* __restrict__ src, int64_t K, int64_t outer,
                                             int64_t ld, const int32_t* __restrict__ zidx, int nz,
                                             int zaxis, uint8_t* __restrict__ codes,
                                             uint8_t* __restrict__ scales,
                                             uint16_t* __restrict__ gathered, int kchunk, int64_t bx,
                                             int64_t by) {
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[kColOut * kColPitch];
  __shared__ __attribute__((aligned(16))) uint8_t s_scales[kColOut * kColBlocks];
  // Extracted lines inside this tile: rows (zero_axis ROWS) as one bit per
  // row of each block, columns one bit per column; with their positions in
  // the index list.
  __shared__ uint32_t s_rmask[kColBlocks];
  __shared__ int32_t s_rpos[kColBlocks * 32];
  __shared__ uint32_t s_cmask[kColOut / 32];
  __shared__ int32_t s_cpos[kColOut];
  const int tid = threadIdx.x;
  const int cg = tid % kColGroups, bi = tid / kColGroups;
  const int64_t cbase = bx * kColOut;
  const int64_t bbase = by * kColBlocks;
  const int64_t c0 = cbase + 4 * cg;
  const int64_t b = bbase + bi;
  const int64_t nblocks = K / 32;
  const bool mine = c0 < outer && b < nblocks;
  const int64_t t0 = b * 32;

  // This thread's share of the index list, loaded before the tile so that
  // waiting for it does not wait for the tile.
  int zv[kMaxK / kColThreads];
#pragma unroll
  for (int q = 0; q < kMaxK / kColThreads; ++q) {
    const int i = tid + q * kColThreads;
    zv[q] = i < nz ? zidx[i] : -1;
  }

  uint32_t w[32][2];
  if (mine) colwise_load<Vec, NT>(w, src, ld, outer, bbase, bi, c0);

  if (tid < kColBlocks) s_rmask[tid] = 0;
  if (tid < kColOut / 32) s_cmask[tid] = 0;
  __syncthreads();
  if (nz > 0) {
    const int64_t lo = zaxis == ADAHOP_AXIS_ROWS ? bbase * 32 : cbase;
    const int span = zaxis == ADAHOP_AXIS_ROWS ? kColBlocks * 32 : kColOut;
#pragma unroll
    for (int q = 0; q < kMaxK / kColThreads; ++q) {
      const int64_t d = (int64_t)zv[q] - lo;
      if (zv[q] >= 0 && d >= 0 && d < span) {
        const int i = tid + q * kColThreads;
        if (zaxis == ADAHOP_AXIS_ROWS) {
          atomicOr(&s_rmask[d / 32], 1u << (d % 32));
          s_rpos[d] = i;
        } else {
          atomicOr(&s_cmask[d / 32], 1u << (d % 32));
          s_cpos[d] = i;
        }
      }
    }
  }
  __syncthreads();

  if (mine) {
    // Extracted lines held by this thread: rows of its block (bit j = row
    // t0 + j) and its own 4 columns (bit q = column c0 + q).
    const uint32_t rmask = s_rmask[bi];
    const uint32_t cbits = (s_cmask[(4 * cg) / 32] >> ((4 * cg) % 32)) & 0xFu;
    // Gather, then clear in the packed words (an extracted element is +0 in
    // the residual). The test is wave-uniform, so waves holding no extracted
    // line skip all of it; a per-lane test would be turned into selects on
    // every word.
    if (__builtin_amdgcn_ballot_w64((rmask | cbits) != 0) != 0) {
      if (gathered) {
        // Rows: gathered [nz][outer]. Registers are indexed by unrolled
        // constants only.
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          if (!((rmask >> j) & 1u)) continue;
          const int64_t p = s_rpos[bi * 32 + j];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (c0 + q < outer)
              gathered[p * outer + c0 + q] = (uint16_t)((w[j][q >> 1] >> (16 * (q & 1))) & 0xFFFFu);
        }
        // Columns: gathered [nz][K], this block's 32 values as 64
        // contiguous bytes.
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (!((cbits >> q) & 1u) || c0 + q >= outer) continue;
          uint32_t pk[16];
#pragma unroll
          for (int j = 0; j < 16; ++j)
            pk[j] = ((w[2 * j][q >> 1] >> (16 * (q & 1))) & 0xFFFFu) |
                    (((w[2 * j + 1][q >> 1] >> (16 * (q & 1))) & 0xFFFFu) << 16);
          uint4* g = reinterpret_cast<uint4*>(gathered + (int64_t)s_cpos[4 * cg + q] * K + t0);
#pragma unroll
          for (int j = 0; j < 4; ++j) g[j] = make_uint4(pk[4 * j], pk[4 * j + 1], pk[4 * j + 2], pk[4 * j + 3]);
        }
      }
      const uint32_t m0 = ((cbits & 1u) ? 0u : 0x0000FFFFu) | ((cbits & 2u) ? 0u : 0xFFFF0000u);
      const uint32_t m1 = ((cbits & 4u) ? 0u : 0x0000FFFFu) | ((cbits & 8u) ? 0u : 0xFFFF0000u);
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const bool z = (rmask >> j) & 1u;
        w[j][0] = z ? 0u : (w[j][0] & m0);
        w[j][1] = z ? 0u : (w[j][1] & m1);
      }
    }
    colwise_quant_to_lds<Had>(w, c0, outer, cg, bi, s_codes, s_scales);
  }
  __syncthreads();

  colwise_write_tile(s_codes, s_scales, codes, scales, kchunk, K, outer, cbase, bbase);
}

// contract ROWS with the outer outlier product formed in the same pass (the
// one-read variant of OE_LEFT / OE_RIGHT). The outlier product needs the
// full bf16 values of the operand FOID does not scan (its rank-k product
// with the extracted lines); when that operand is quantized down its
// columns, these tiles form the product while the values are in registers
// for the quantization, so the operand is read from memory once instead of
// twice:
//   P_s[c][p] = sum over t in group s of src[t][c] * lines[p][t]
// (lines: the k extracted lines, bf16 [k][K]), fp32, for every column c and
// p < k <= 64, written to partials[s] ([outer][k], or [k][outer] with
// ByLine); the groups are then summed in order by the outlier product's
// reduction.
// Tiles as colwise_tile's (256 columns x 4 blocks of 32), but wave w holds
// columns 64 w .. 64 w + 63 of all 4 blocks: lane l takes the 4 columns
// 64 w + 4 (l % 16) .. + 3 of block l / 16, so the 16 lanes of a lane group
// hold 16 consecutive column groups at the same rows. That is the layout of
// a v_mfma_f32_16x16x32_bf16 operand (lane l: matrix row l % 16, 8
// consecutive k of k-group l / 16): with column q of each lane's group as the
// row and 8 consecutive rows of its block as the k values, the raw bf16
// words form the first operand after one byte permutation per dword; lane l
// loads the matching 8 values of line 16 pb + l % 16 as the second. A
// workgroup walks `tiles_per_wg` consecutive tiles down its columns (group
// `by`) with the 16 accumulator blocks (4 column offsets q x 4 line blocks
// pb) in registers, then writes its group's partial sums once.
typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
typedef float v4f32 __attribute__((ext_vector_type(4)));
constexpr int kFusedOeMaxK = 64;

template <bool Vec, bool ByLine>
__device__ __forceinline__ void colwise_oe_tiles(const uint16_t* __restrict__ src, int64_t K,
                                                 int64_t outer, int64_t ld,
                                                 uint8_t* __restrict__ codes,
                                                 uint8_t* __restrict__ scales, int kchunk,
                                                 const uint16_t* __restrict__ lines, int k,
                                                 int tiles_per_wg, float* __restrict__ partials,
                                                 int64_t bx, int64_t by) {
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[kColOut * kColPitch];
  __shared__ __attribute__((aligned(16))) uint8_t s_scales[kColOut * kColBlocks];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cg = wave * 16 + (lane & 15), bi = lane >> 4;
  const int64_t cbase = bx * kColOut;
  const int64_t c0 = cbase + 4 * cg;
  const int64_t nblocks = K / 32;
  const int64_t ntiles = (nblocks + kColBlocks - 1) / kColBlocks;
  const int64_t tt0 = by * tiles_per_wg;
  const int64_t tt1 = tt0 + tiles_per_wg < ntiles ? tt0 + tiles_per_wg : ntiles;
  const int npb = (k + 15) / 16;

  v4f32 acc[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) acc[q][pb] = v4f32{0.0f, 0.0f, 0.0f, 0.0f};

  for (int64_t tt = tt0; tt < tt1; ++tt) {
    const int64_t bbase = tt * kColBlocks;
    const int64_t b = bbase + bi;
    const bool mine = c0 < outer && b < nblocks;
    const int64_t t0 = b * 32;
    uint32_t w[32][2];
    if (mine) {
      colwise_load<Vec, true>(w, src, ld, outer, bbase, bi, c0);
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) { w[j][0] = 0u; w[j][1] = 0u; }
    }
    // Second operands: line p = 16 pb + l % 16 at rows t0 + 8 st .. + 7.
    uint4 lf[4][4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) {
        const int p = 16 * pb + (lane & 15);
        lf[st][pb] = make_uint4(0, 0, 0, 0);
        if (pb < npb && p < k && b < nblocks)
          lf[st][pb] = *reinterpret_cast<const uint4*>(lines + (int64_t)p * K + t0 + 8 * st);
      }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // Column c0 + q at rows t0 + 8 st .. + 7, two bf16 per dword.
        const int h = q >> 1;
        uint32_t a[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t lo = w[8 * st + 2 * d][h], hi = w[8 * st + 2 * d + 1][h];
          a[d] = (q & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        }
        const v8bf16 fa = __builtin_bit_cast(v8bf16, make_uint4(a[0], a[1], a[2], a[3]));
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
          if (pb >= npb) continue;
          acc[q][pb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              fa, __builtin_bit_cast(v8bf16, lf[st][pb]), acc[q][pb], 0, 0, 0);
        }
      }
    }
    if (mine) colwise_quant_to_lds<true>(w, c0, outer, cg, bi, s_codes, s_scales);
    __syncthreads();
    colwise_write_tile(s_codes, s_scales, codes, scales, kchunk, K, outer, cbase, bbase);
    __syncthreads();   // the next tile reuses the LDS rows
  }

  // Accumulator block (q, pb), register v of lane l: matrix row 4 (l / 16) + v
  // (column 64 w + 4 row + q), line 16 pb + l % 16.
  float* P = partials + by * outer * k;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      if (pb >= npb) continue;
      const int p = 16 * pb + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t c = cbase + 64 * wave + 16 * (lane >> 4) + 4 * v + q;
        if (c < outer && p < k) {
          if (ByLine) P[(int64_t)p * outer + c] = acc[q][pb][v];
          else P[c * k + p] = acc[q][pb][v];
        }
      }
    }
}

}  // namespace
}  // namespace adahop
