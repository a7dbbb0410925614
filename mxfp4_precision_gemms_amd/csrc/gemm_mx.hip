// Fused MXFP4 + BF16 GEMM and scatter-add for gfx950.
//
// "AdaHOP ..." (arXiv 2604.02525), appendix kernels 3 and 4: the residual
// product runs in MXFP4 while the outlier product runs in bf16, and the
// outlier result is added into the residual result in place, without a
// separate pass over the output.
//
// Residual product: CDNA4 scaled FP4 matrix cores,
//   v_mfma_scale_f32_32x32x64_f8f6f4 (both operands E2M1, one E8M0 scale byte
//   per lane = per 32-element K block). Lane l of a wave supplies row l%32 of
//   the 32x64 A block (B: column l%32), K half l/32: 16 bytes of packed codes,
//   exactly one 32-element MX block, plus that block's scale byte.
// Tiling: a workgroup computes a 256 x 256 tile of C: in the main kernel 8
//   waves of 128 x 64 (4 x 2 MFMA blocks, 128 fp32 accumulators per lane),
//   two per SIMD; in the fallback kernel 4 waves of 128 x 128. Workgroup ids
//   are remapped so that each XCD works through a contiguous range of tiles,
//   8 tile-rows high, whose operand rows its L2 shares.
// Main kernel (gemm_mx_ring8_kernel, K % 512 == 0): K advances 128 elements
//   per stage through a 4-slot LDS ring filled by direct global->LDS buffer
//   loads up to three stages ahead, a stage's loads spread over the MFMAs
//   between two workgroup barriers; the scales come K-chunked from the quantizers
//   or from a stage-major copy made just before (scale_stage_kernel). One
//   workgroup runs per CU; a last round of tiles that would leave more than
//   half of the 256 CUs idle is split along K, and gemm_split_fixup_kernel
//   adds the parts. Other K: gemm_mx_kernel, 256-element stages double
//   buffered in LDS with register-staged buffer loads.
// Outlier product: bf16 matrix cores (v_mfma_f32_32x32x16_bf16), 128 x 64
//   tiles, K split across workgroups into fp32 partials that a small kernel
//   sums in a fixed order; the FP4 kernel's epilogue adds a line's reduced
//   outlier product to the fp32 accumulators before the single rounding to
//   the output type (the scatter-add). Inner extraction (a rank-k term on
//   every output) runs as extra bf16 MFMAs on the tile's own accumulators.
//   No atomics: results are deterministic.
#include <mutex>
#include <utility>

#include "adahop_internal.h"

namespace adahop {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s16 __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

// gfx950 converts to bf16 in hardware, rounding to nearest even (finite
// inputs; the tests check it against the integer rounding rule).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Two values in one conversion: a in the low half, b in the high half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 p = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

// Row of a 32x32 MFMA accumulator held in register v by lane l (column l%32).
__device__ __forceinline__ int acc_row(int v, int lane) {
  return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

// Calls f(std::integral_constant<int, 0>) ... f(<N-1>): loops whose index
// must be a compile-time constant (register arrays stay in registers).
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------------------
// FP4 GEMM
// ---------------------------------------------------------------------------
constexpr int BM = 256, BN = 256;
constexpr int BKB = 128;                // bytes of packed codes per row per stage (256 elements)
constexpr int SCB = BKB / 16;           // scale bytes per row per stage (8)
constexpr int LROW = BKB + 16;          // LDS row stride: 144 bytes (9 x 16, odd)
constexpr int kGemmThreads = 256;
constexpr int WM = 128, WN = 128;       // wave sub-tile (2 x 2 waves)
constexpr int FM = WM / 32, FN = WN / 32;
constexpr int kLdsA = BM * LROW, kLdsB = BN * LROW;
constexpr int kChunksA = BM * BKB / 16 / kGemmThreads;   // 16-byte chunks per thread per stage
constexpr int kChunksB = BN * BKB / 16 / kGemmThreads;
constexpr int kRowsPerPass = kGemmThreads / (BKB / 16);  // rows one pass of the workgroup copies
constexpr int kGroupM = 8;              // tile rows that run together on one XCD
constexpr int kBufferFlags = 0x00020000;   // raw buffer descriptor word 3 (gfx9 family)

struct GemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const uint32_t* a_sst;        // stage-major scale copies (main kernel): [K/128][m] words
  const uint32_t* b_sst;        //   and [K/128][n] words
  int64_t m, n, K;
  void* C;
  int64_t ldc;
  int out_f32;
  int tiles_m, tiles_n;
  // Last round split along K (main kernel): work items from split_full on
  // each take 1 / split_parts of K of one of the split_count tiles from
  // split_full on and leave their fp32 sums in split_ws ([tile][part][256 x
  // 256]); gemm_split_fixup_kernel adds the parts and runs the epilogue.
  int split_full, split_count, split_parts;   // whole tiles, split tiles, parts per split tile
  float* split_ws;
  // outlier epilogue
  int oe_mode;
  int oe_k;
  const int32_t* oe_idx;
  const float* oe_p;            // reduced outlier product: OE_LEFT [k][n], OE_RIGHT [m][k]
  int vec_ok;                   // C rows allow 16-byte stores (ldc % 4 fp32 / % 8 bf16, C aligned)
  const uint16_t* ia_ptr; int64_t ia_ld; int ia_inner;   // OE_INNER a: (i, p)
  const uint16_t* ib_ptr; int64_t ib_ld; int ib_inner;   // OE_INNER b: (j, p)
  // bf16 operands stored across K ([K][ld], ring kernel): bytes per stored row
  int64_t a_ldb, b_ldb;
  // Outer outlier product run inside the main kernel (OE_LEFT / OE_RIGHT with
  // oe_items > 0): item e computes, for the 256-wide block e % oe_tiles_w of
  // the operand stored across K ("wide": A for OE_RIGHT, B for OE_LEFT) and
  // K-part e / oe_tiles_w (oe_kst bf16 stages of 32), the partial sums
  // P_s(w, p) = sum_t wide(w, t) line(p, t) of its <= 64 lines, written to
  // oe_part ([s][w][p] for OE_RIGHT, [s][p][w] for OE_LEFT, fp32). The tile
  // epilogues then leave C's extracted lines to oe_scatter_kernel and keep
  // their fp32 residual there in oe_res ([w][p] / [p][w]).
  int oe_items, oe_tiles_w, oe_kst;
  const uint8_t* oe_wide;
  int64_t oe_wide_ldb, oe_wide_n;
  const uint8_t* oe_lines;       // [k][K] bf16
  float* oe_part;
  float* oe_res;
};

__device__ __forceinline__ int lower_bound_i32(const int32_t* idx, int n, int64_t v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)idx[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ uint16_t view_at(const uint16_t* p, int64_t ld, int inner, int64_t r,
                                            int64_t t) {
  return inner ? p[r * ld + t] : p[t * ld + r];
}

// Logical position of workgroup `bid` among `count` workgroups. The hardware
// deals workgroups round-robin to the 8 XCDs (bid % 8); each XCD gets a
// contiguous band of the logical order.
__device__ __forceinline__ int xcd_band(int bid, int count) {
  return count % 8 == 0 ? (bid & 7) * (count / 8) + (bid >> 3) : bid;
}

// Tile at logical position pid: the logical order walks groups of kGroupM
// tile rows column by column, so the ~32 tiles an XCD runs at once form an
// 8 x 4 block that shares operand rows in that XCD's L2 (8 rows measured
// 1.3 % faster than 4 on the 32768 x 14336 x 4096 forward, the same
// elsewhere).
__device__ __forceinline__ void tile_at(int pid, int tiles_m, int tiles_n, int* tm, int* tn) {
  const int per_group = kGroupM * tiles_n;
  const int group = pid / per_group;
  const int first_m = group * kGroupM;
  const int gm = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  const int in_group = pid - group * per_group;
  *tm = first_m + in_group % gm;
  *tn = in_group / gm;
}

__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int* tm, int* tn) {
  tile_at(xcd_band(bid, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
}

// Inner-extraction term and epilogue, shared by both GEMM kernels. `acc` is
// the wave's 128 x 128 sub-tile of the tile at (m0, n0), computed as C^T
// blocks: the MFMA's first operand holds B rows (C columns) and its second A
// rows (C rows), so lane l of block (I, J) holds C row 32 I + l%32 and, in
// registers 4 G .. 4 G + 3, the four consecutive C columns 32 J + 8 G +
// 4 (l/32) .. +3 -- one 8-byte bf16 (16-byte fp32) store each.
// Epilogue of a workgroup of THREADS threads whose wave w holds the TFM x TFN
// 32x32 blocks at rows (w / WAVES_N) * TWM, columns (w % WAVES_N) * TWN of
// the tile, in C^T register layout (lane l: row l % 32; register 4 G + e:
// column 8 G + 4 (l / 32) + e of the block).
template <int TFM, int TFN, int TWM, int TWN, int WAVES_N>
__device__ __forceinline__ void gemm_inner_term(const GemmArgs& g, v16f (&acc)[TFM][TFN], int64_t m0,
                                                int64_t n0) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lrow = lane & 31, khalf = lane >> 5;
  // Inner extraction: C += a[:, 0:k] * b[:, 0:k]^T on bf16 matrix cores,
  // 16 extracted lines per MFMA (lane: row l%32, lines 8*(l/32) .. +7).
  if (g.oe_mode == ADAHOP_ROUTE_OE_INNER) {
    for (int p0 = 0; p0 < g.oe_k; p0 += 16) {
      v8bf fa[TFM], fb[TFN];
#pragma unroll
      for (int i = 0; i < TFM; ++i) {
        int64_t row = m0 + wm * TWM + i * 32 + lrow;
        row = row < g.m ? row : g.m - 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int p = p0 + 8 * khalf + e;
          const uint16_t h = p < g.oe_k ? view_at(g.ia_ptr, g.ia_ld, g.ia_inner, row, p) : 0;
          fa[i][e] = __builtin_bit_cast(__bf16, h);
        }
      }
#pragma unroll
      for (int j = 0; j < TFN; ++j) {
        int64_t col = n0 + wn * TWN + j * 32 + lrow;
        col = col < g.n ? col : g.n - 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int p = p0 + 8 * khalf + e;
          const uint16_t h = p < g.oe_k ? view_at(g.ib_ptr, g.ib_ld, g.ib_inner, col, p) : 0;
          fb[j][e] = __builtin_bit_cast(__bf16, h);
        }
      }
      static_for<TFM>([&](auto I) {
        static_for<TFN>([&](auto J) {
          acc[I][J] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[J], fa[I], acc[I][J], 0, 0, 0);
        });
      });
    }
  }
}

// Outer-extraction scatter-add, one rounding to the output type, stores.
template <int TFM, int TFN, int TWM, int TWN, int WAVES_N, int THREADS>
__device__ __forceinline__ void gemm_store(const GemmArgs& g, v16f (&acc)[TFM][TFN], int64_t m0,
                                           int64_t n0, int* s_pos) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lrow = lane & 31, khalf = lane >> 5;
  // Outer extraction: positions of this tile's extracted rows / columns.
  const bool oe_rows = g.oe_mode == ADAHOP_ROUTE_OE_LEFT;
  const bool oe_cols = g.oe_mode == ADAHOP_ROUTE_OE_RIGHT;
  bool any_oe = false;
  if (oe_rows || oe_cols) {
    const int64_t lo_v = oe_rows ? m0 : n0;
    const int64_t span = oe_rows ? BM : BN;
    const int lo = lower_bound_i32(g.oe_idx, g.oe_k, lo_v);
    const int hi = lower_bound_i32(g.oe_idx, g.oe_k, lo_v + span);
    any_oe = hi > lo;
    if (any_oe) {
      for (int q = tid; q < span; q += THREADS) s_pos[q] = -1;
      __syncthreads();
      for (int p = lo + tid; p < hi; p += THREADS) s_pos[g.oe_idx[p] - lo_v] = p;
      __syncthreads();
    }
  }

  // Addresses: one row pointer per 32-row block I (the only 64-bit products);
  // within a block every store is that pointer plus a constant offset.
  const bool full = m0 + BM <= g.m && n0 + BN <= g.n && g.vec_ok;
  const int lc0 = wn * TWN + 4 * khalf;                 // tile column of (J, G) = lc0 + 32 J + 8 G
  const int64_t col0 = n0 + lc0;
  static_for<TFM>([&](auto I) {
    const int lr = wm * TWM + I * 32 + lrow;
    const int64_t row = m0 + lr;
    const int prow = (any_oe && oe_rows) ? s_pos[lr] : -1;
    // Outlier product values for this row: OE_LEFT its extracted row's
    // values from column col0 on, OE_RIGHT its row of k values. With the
    // product computed inside the kernel (oe_res), the residual of the
    // extracted lines goes to oe_res instead, for oe_scatter_kernel.
    const float* oe_row = nullptr;
    float* res_row = nullptr;
    if (any_oe && row < g.m) {
      if (g.oe_res) {
        if (oe_rows) { if (prow >= 0) res_row = g.oe_res + (int64_t)prow * g.n + col0; }
        else res_row = g.oe_res + row * g.oe_k;
      } else if (oe_rows) {
        if (prow >= 0) oe_row = g.oe_p + (int64_t)prow * g.n + col0;
      } else {
        oe_row = g.oe_p + row * g.oe_k;
      }
    }
    const int64_t off = row * g.ldc + col0;
    float* cf = static_cast<float*>(g.C) + off;
    uint16_t* cb = static_cast<uint16_t*>(g.C) + off;
    static_for<TFN>([&](auto J) {
      float v[4][4];
      static_for<4>([&](auto G) {
        constexpr int dc = 32 * decltype(J)::value + 8 * decltype(G)::value;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[G][e] = acc[I][J][4 * G + e];
        if (oe_row != nullptr) {
          // scatter-add of the outlier product (the residual there is 0)
          if (oe_rows) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (col0 + dc + e < g.n) v[G][e] += oe_row[dc + e];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int p = lc0 + dc + e < BN ? s_pos[lc0 + dc + e] : -1;
              if (p >= 0) v[G][e] += oe_row[p];
            }
          }
        } else if (res_row != nullptr) {
          if (oe_rows) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (col0 + dc + e < g.n) res_row[dc + e] = v[G][e];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int p = lc0 + dc + e < BN ? s_pos[lc0 + dc + e] : -1;
              if (p >= 0) res_row[p] = v[G][e];
            }
          }
        }
      });
      if (full && !g.out_f32) {
        // Lanes l and l + 32 hold the same row, column quads 8 G and 8 G + 4:
        // one swap of half-waves per pair of quads gives lane l columns
        // 16 P .. +7 and lane l + 32 columns 16 P + 8 .. +15, so each lane
        // stores 16 contiguous bytes (2.4x fewer store cycles than 8-byte
        // pieces, measured).
        uint16_t* cbs = cb + 4 * khalf;                 // row pointer at column n0 + wn * TWN + 8 khalf
        static_for<2>([&](auto P) {
          constexpr int q = 2 * decltype(P)::value;
          const auto a = __builtin_amdgcn_permlane32_swap(pack_bf16x2(v[q][0], v[q][1]),
                                                          pack_bf16x2(v[q + 1][0], v[q + 1][1]), false, false);
          const auto b = __builtin_amdgcn_permlane32_swap(pack_bf16x2(v[q][2], v[q][3]),
                                                          pack_bf16x2(v[q + 1][2], v[q + 1][3]), false, false);
          *reinterpret_cast<uint4*>(cbs + 32 * decltype(J)::value + 16 * decltype(P)::value) =
              make_uint4(a[0], b[0], a[1], b[1]);
        });
      } else {
        static_for<4>([&](auto G) {
          constexpr int dc = 32 * decltype(J)::value + 8 * decltype(G)::value;
          if (full) {
            *reinterpret_cast<float4*>(cf + dc) = make_float4(v[G][0], v[G][1], v[G][2], v[G][3]);
          } else if (row < g.m) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (col0 + dc + e >= g.n) continue;
              if (g.out_f32)
                cf[dc + e] = v[G][e];
              else
                cb[dc + e] = f32_to_bf16_rne(v[G][e]);
            }
          }
        });
      }
    });
  });
}

template <int TFM, int TFN, int TWM, int TWN, int WAVES_N, int THREADS>
__device__ __forceinline__ void gemm_finish(const GemmArgs& g, v16f (&acc)[TFM][TFN], int64_t m0,
                                            int64_t n0, int* s_pos) {
  gemm_inner_term<TFM, TFN, TWM, TWN, WAVES_N>(g, acc, m0, n0);
  gemm_store<TFM, TFN, TWM, TWN, WAVES_N, THREADS>(g, acc, m0, n0, s_pos);
}

// One stage of global data held in registers between its load and its LDS store.
struct Stage {
  uint4 a[kChunksA], b[kChunksB];
  uint2 sa, sb;
};

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// Register-staged kernel for any K % 32 == 0 (stages of 256 K-elements, the
// last one masked). KAligned: K % 256 == 0 and 8-byte aligned scale rows.
template <bool KAligned>
__global__ void __launch_bounds__(kGemmThreads, 1) gemm_mx_kernel(GemmArgs g) {
  // LDS rows are 144 bytes apart: 16-byte chunk c of row r starts at byte
  // 144 r + 16 c, so the 16-byte units that 8 (or 16) consecutive rows touch
  // at one chunk are 9 r + c mod 8 (mod 16): all distinct, no bank conflicts,
  // and a fragment's address differs between K-steps only by an immediate.
  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][kLdsA];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2][kLdsB];
  __shared__ __attribute__((aligned(8))) uint8_t s_sa[2][BM * SCB];
  __shared__ __attribute__((aligned(8))) uint8_t s_sb[2][BN * SCB];
  __shared__ int s_pos[BM > BN ? BM : BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(blockIdx.x, g.tiles_m, g.tiles_n, &tm, &tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t Kb = g.K / 2;          // bytes per packed row
  const int64_t Ks = g.K / 32;         // scale bytes per row
  const int nk = (int)((Kb + BKB - 1) / BKB);
  const int rows_a = (int)(g.m - m0 < BM ? g.m - m0 : BM);
  const int rows_b = (int)(g.n - n0 < BN ? g.n - n0 : BN);

  // Buffer descriptors over this tile's rows: loads past the last row read 0.
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(g.a_codes + m0 * Kb), 0, (int)(rows_a * Kb), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(g.b_codes + n0 * Kb), 0, (int)(rows_b * Kb), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(g.a_scales + m0 * Ks), 0, (int)(rows_a * Ks), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(g.b_scales + n0 * Ks), 0, (int)(rows_b * Ks), kBufferFlags);

  // Copy pattern: chunk (tid % 8) of rows tid / 8 + 32 i, so 8 lanes read one
  // row's 128 contiguous bytes.
  const int c_ld = tid & 7;
  const int r_ld = tid >> 3;
  const int voff0 = r_ld * (int)Kb + c_ld * 16;
  const int vstep = kRowsPerPass * (int)Kb;

  auto load_scales = [&](__amdgpu_buffer_rsrc_t rs, int64_t sb0) -> uint2 {
    if (KAligned) {
      const v2u w = __builtin_amdgcn_raw_buffer_load_b64(rs, tid * (int)Ks, (int)sb0, 0);
      return make_uint2(w.x, w.y);
    }
    // K tail: byte loads, bytes past K read as 0 (their codes are 0 too).
    uint32_t v[2] = {0, 0};
#pragma unroll
    for (int q = 0; q < SCB; ++q) {
      const bool in = sb0 + q < Ks;
      const uint32_t b = __builtin_amdgcn_raw_buffer_load_b8(rs, tid * (int)Ks + (int)(in ? sb0 + q : 0), 0, 0);
      v[q >> 2] |= (in ? b : 0u) << (8 * (q & 3));
    }
    return make_uint2(v[0], v[1]);
  };
  auto load_stage = [&](Stage& st, int kt) {
    const int64_t kb0 = (int64_t)kt * BKB;
    const bool kin = KAligned || kb0 + c_ld * 16 < Kb;
    const int kc = kin ? (int)kb0 : 0;
#pragma unroll
    for (int i = 0; i < kChunksA; ++i) {
      const v4u q = __builtin_amdgcn_raw_buffer_load_b128(ra, voff0 + i * vstep, kc, 0);
      st.a[i] = kin ? make_uint4(q.x, q.y, q.z, q.w) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kChunksB; ++i) {
      const v4u q = __builtin_amdgcn_raw_buffer_load_b128(rb, voff0 + i * vstep, kc, 0);
      st.b[i] = kin ? make_uint4(q.x, q.y, q.z, q.w) : make_uint4(0, 0, 0, 0);
    }
    st.sa = load_scales(rsa, (int64_t)kt * SCB);
    st.sb = load_scales(rsb, (int64_t)kt * SCB);
  };
  const int w_off = r_ld * LROW + c_ld * 16;     // this thread's LDS store offset (pass 0)
  auto store_stage = [&](const Stage& st, int buf) {
#pragma unroll
    for (int i = 0; i < kChunksA; ++i)
      *reinterpret_cast<uint4*>(&s_a[buf][w_off + i * kRowsPerPass * LROW]) = st.a[i];
#pragma unroll
    for (int i = 0; i < kChunksB; ++i)
      *reinterpret_cast<uint4*>(&s_b[buf][w_off + i * kRowsPerPass * LROW]) = st.b[i];
    *reinterpret_cast<uint2*>(&s_sa[buf][tid * SCB]) = st.sa;
    *reinterpret_cast<uint2*>(&s_sb[buf][tid * SCB]) = st.sb;
  };

  v16f acc[FM][FN];
  static_for<FM>([&](auto I) {
    static_for<FN>([&](auto J) {
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[I][J][v] = 0.0f;
    });
  });

  const int lrow = lane & 31, khalf = lane >> 5;
  const int fa_off = (wm * WM + lrow) * LROW + khalf * 16;   // fragment i, K-step ks: + 32 LROW i + 32 ks
  const int fb_off = (wn * WN + lrow) * LROW + khalf * 16;
  const int sa_off = (wm * WM + lrow) * SCB;
  const int sb_off = (wn * WN + lrow) * SCB;
  // One stage: 4 K-steps of 64. Lane (row l%32, half l/32) of K-step ks reads
  // chunk 2 ks + half of its row and scale byte 2 ks + half; each row's 8
  // scale bytes are read once per stage and pre-shifted by 8 * half, so the
  // MFMA's opsel picks byte 2 (ks % 2) of dword ks / 2.
  auto compute = [&](int buf) {
    const uint8_t* pa = &s_a[buf][fa_off];
    const uint8_t* pb = &s_b[buf][fb_off];
    uint2 sca[FM], scb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const uint2 w = *reinterpret_cast<const uint2*>(&s_sa[buf][sa_off + i * 32 * SCB]);
      sca[i] = make_uint2(w.x >> (8 * khalf), w.y >> (8 * khalf));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const uint2 w = *reinterpret_cast<const uint2*>(&s_sb[buf][sb_off + j * 32 * SCB]);
      scb[j] = make_uint2(w.x >> (8 * khalf), w.y >> (8 * khalf));
    }
    static_for<4>([&](auto KS) {
      v8i fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint4 q = *reinterpret_cast<const uint4*>(pa + i * 32 * LROW + 32 * KS);
        fa[i] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint4 q = *reinterpret_cast<const uint4*>(pb + j * 32 * LROW + 32 * KS);
        fb[j] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      }
      constexpr int kSel = 2 * (KS % 2);
      static_for<FM>([&](auto I) {
        static_for<FN>([&](auto J) {
          const int sa_w = KS < 2 ? (int)sca[I].x : (int)sca[I].y;
          const int sb_w = KS < 2 ? (int)scb[J].x : (int)scb[J].y;
          acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fb[J], fa[I], acc[I][J], 4, 4, kSel, sb_w, kSel, sa_w);
        });
      });
    });
  };

  // Pipeline: stage kt+1's global loads are in flight in registers while
  // stage kt feeds the matrix cores from LDS; they go to the other LDS slot
  // after this stage's MFMAs are issued.
  Stage st;
  load_stage(st, 0);
  store_stage(st, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_stage(st, kt + 1);
    compute(buf);
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) store_stage(st, buf ^ 1);
    __syncthreads();
  }

  gemm_finish<FM, FN, WM, WN, 2, kGemmThreads>(g, acc, m0, n0, s_pos);
}


// ---------------------------------------------------------------------------
// Main kernel for K % 512 == 0 (gemm_mx_ring8_kernel): a 4-slot LDS ring
// filled by direct global->LDS buffer loads (no staging registers), up to
// three stages ahead of the matrix cores. Stage = 128 K-elements: A and B 256 rows x
// 64 bytes each plus 4 scale bytes per row. Before a stage is read, every
// wave waits until only its loads of the two later stages are in flight, then
// the workgroup barrier publishes the stage. LDS rows of 64 bytes keep their
// four 16-byte chunks XOR-swizzled by ((r >> 1) ^ (r >> 2)) & 3, so a wave's
// fragment reads of 8 (or 16) consecutive rows hit distinct banks.
// ---------------------------------------------------------------------------
constexpr int RBK = 64;                       // bytes per row per stage
constexpr int kRingSlots = 4;
constexpr int kSlotA = BM * RBK, kSlotB = BN * RBK;   // 16 KB each

// One LDS object per slot: the compiler's alias analysis then sees that the
// loads in flight into one slot do not touch the slot being read, and adds no
// wait for them before the reads.
struct RingSlot {
  uint8_t a[kSlotA];
  uint8_t b[kSlotB];
  uint8_t sa[BM * 4];
  uint8_t sb[BN * 4];
};
__shared__ __attribute__((aligned(1024))) RingSlot g_ring0;
__shared__ __attribute__((aligned(1024))) RingSlot g_ring1;
__shared__ __attribute__((aligned(1024))) RingSlot g_ring2;
__shared__ __attribute__((aligned(1024))) RingSlot g_ring3;
__shared__ int g_ring_pos[BM > BN ? BM : BN];

template <int S>
__device__ __forceinline__ RingSlot& ring_slot() {
  if constexpr (S == 0) return g_ring0;
  else if constexpr (S == 1) return g_ring1;
  else if constexpr (S == 2) return g_ring2;
  else return g_ring3;
}

// s_waitcnt immediate (gfx9 encoding): vmcnt bits [3:0] and [15:14], expcnt
// [6:4] (7 = no wait), lgkmcnt [11:8].
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

__device__ __forceinline__ int ring_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// A buffer offset past the end of every buffer the main kernel reads (their
// sizes stay below 2^31 - 16): such a load returns 0 without touching memory.
constexpr int kPastEnd = 0x7FFFFFF0;

typedef __attribute__((address_space(3))) void lds_void;

// ---------------------------------------------------------------------------
// 8 waves, two per SIMD: wave w computes rows
// 128 (w / 4) .. +127, columns 64 (w % 4) .. +63 of the 256 x 256 tile (4 x 2
// MFMA blocks, 128 accumulators), so while one wave of a SIMD waits -- for a
// load to be accepted by the memory pipeline or for an LDS read -- the other
// keeps the matrix core busy. Each wave copies an eighth of a stage with 5
// loads: 16 rows each of A and B twice (1 KB per load), and a quarter of the
// A scales (waves 0-3) or of the B scales (waves 4-7). Fragments are double
// buffered per K-step: the second K-step's are read during the first one's
// MFMAs, the next stage's first K-step's during the second one's.
// ---------------------------------------------------------------------------
constexpr int kRing8Threads = 512;
constexpr int R8_FM = 4, R8_FN = 2, R8_WM = 128, R8_WN = 64;
constexpr int kLoads8PerStage = 5;            // per wave

// A split tile's part in the workspace: a row-major fp32 256 x 256 matrix.
constexpr int kSplitPartF4 = BM * BN / 4;      // float4 per part (256 KB)

// One work item: a whole tile, or one K-part of a split tile of the last round.
struct RingItem {
  int tm, tn;
  int part, split_tile;          // part < 0: a whole tile
  int kt0, kt1;                  // K stages [kt0, kt1), a multiple of 4 apart
  int64_t m0, n0;
  __amdgpu_buffer_rsrc_t ra, rb;
  int voffa[2], voffb[2], soff;
};

// Persistent: one workgroup per CU (gridDim.x <= number of items) takes the
// work items r * gridDim.x + p(b), r = 0, 1, ..., where p spreads each round
// over the XCDs in contiguous bands (xcd_band). Whole tiles come first, the
// split parts of the last round after them. Before a tile's epilogue the
// next item's first stages (three, and two of the fourth's loads) are
// already in flight, so the ring refills while the accumulators are stored.
//
// Bf16: the operands are plain bf16 rows (A [m, K], B [n, K], row stride K),
// no scales. A 64-byte stage row is then 32 elements and a 16-byte fragment
// is the 8 bf16 that v_mfma_f32_32x32x16_bf16 takes per lane (k = 8 (l / 32)
// .. +7 of a 16-deep step) -- the FP4 fragment's place in the row, so the
// ring, the swizzle and the fragment reads are the same; each wave issues 4
// loads per stage instead of 5.
//
// TA / TB (bf16 only): that operand is stored across K, [K][ld] with the
// tile's 256 rows (of C) contiguous. A slot then holds 32 K-rows of 512
// bytes; LDS-DMA load j of wave w fills K-rows 2 (2 w + j) + l / 32, lane l
// putting logical 16-byte chunk (l % 32) ^ 4 h(k) at physical chunk l % 32,
// h(k) = (k & 3) | ((k >> 3) & 1) << 2. A fragment is two
// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// t of its result from the 4 elements at the address of lane 4 t + i / 4,
// element i % 4. Lane L of group G addresses K-row 8 (G / 2) + 4 r + L / 4
// (read r = 0, 1) and the 4 columns 16 (G % 2) + 4 (L % 4) .. +3 of the
// 32-column block, so lane 16 G + i receives column 16 (G % 2) + i, K-rows
// 8 (G / 2) + 4 r .. +3: the MFMA's layout. The swizzle puts the 8 K-rows
// one read touches in 8 different 64-byte column groups.
template <bool Chunked, bool Bf16, bool TA = false, bool TB = false>
__global__ void __launch_bounds__(kRing8Threads, 1) gemm_mx_ring8_kernel(GemmArgs g) {
  static_assert(!(Chunked && Bf16), "bf16 operands come in rows");
  static_assert(Bf16 || (!TA && !TB), "only bf16 operands are read across K");
  constexpr int kLoads = Bf16 ? 4 : kLoads8PerStage;   // per wave per stage
  // LDS reads per K-step: fragments (two per operand block stored across K)
  // and, for FP4, the scale words.
  constexpr int kDs = (TA ? 2 : 1) * R8_FM + (TB ? 2 : 1) * R8_FN + (Bf16 ? 0 : R8_FM + R8_FN);
  // K-step 1 reads no scales: a lane's 16 bits of a row's stage scale word
  // hold both K-steps' scales, read once with K-step 0.
  constexpr int kDs1 = (TA ? 2 : 1) * R8_FM + (TB ? 2 : 1) * R8_FN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Wave-uniform (scalar): the scale loads below pick their descriptor by it.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t Kb = Bf16 ? g.K * 2 : g.K / 2;         // bytes per row
  const int64_t Ks = g.K / 32;
  const int nk = (int)(Kb / RBK);
  const int items = g.split_full + g.split_count * g.split_parts;
  const int G = gridDim.x, bid = blockIdx.x;

  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(g.a_sst), 0, (int)(g.m * Ks), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(g.b_sst), 0, (int)(g.n * Ks), kBufferFlags);
  // Load j (0, 1) of this wave fills LDS bytes [1024 (2 wave + j), +1024) of
  // a slot: rows 16 (2 wave + j) + lane / 4, physical chunk lane % 4 holding
  // logical chunk (lane % 4) ^ swz(row).
  const int row0 = 32 * wave + (lane >> 2);
  const int chunk = (lane & 3) ^ ring_swz(row0);    // swz is the same for rows row0 + 16 j
  const int stage_a = TA ? 32 * (int)g.a_ldb : Chunked ? (int)g.m * RBK : RBK;
  const int stage_b = TB ? 32 * (int)g.b_ldb : Chunked ? (int)g.n * RBK : RBK;
  // Operand stored across K: this lane's load j offset within a stage, or
  // past the end of the buffer when its 16-byte chunk (8 columns; ld is a
  // multiple of 8) starts at or beyond the operand's last column, so that a
  // ragged tile reads nothing outside the operand whatever K-row it is on.
  auto tr_voff = [&](int j, int64_t ldb, int64_t c0) {
    const int k = 2 * (2 * wave + j) + (lane >> 5);
    const int h = (k & 3) | (((k >> 3) & 1) << 2);
    const int chunk = (lane & 31) ^ (4 * h);
    return 8 * (int64_t)chunk < ldb / 2 - c0 ? k * (int)ldb + 16 * chunk : kPastEnd;
  };
  // Scales: waves 0-3 copy A rows 64 (w % 4) + lane, waves 4-7 B rows.
  const bool sc_a = wave < 4;
  const int srow = 64 * (wave & 3) + lane;
  const int sstage = sc_a ? (int)(g.m * 4) : (int)(g.n * 4);

  // Item of round r for this workgroup, or -1.
  auto item_of = [&](int r) {
    const int base = r * G;
    if (base >= items) return -1;
    const int cnt = items - base < G ? items - base : G;
    return bid < cnt ? base + xcd_band(bid, cnt) : -1;
  };
  auto setup = [&](int item) {
    RingItem it;
    int tm, tn, part = -1, split_tile = 0;
    if (item < g.split_full) {
      tile_at(item, g.tiles_m, g.tiles_n, &tm, &tn);
    } else {
      const int t = item - g.split_full;
      split_tile = t / g.split_parts;
      part = t % g.split_parts;
      tile_at(g.split_full + split_tile, g.tiles_m, g.tiles_n, &tm, &tn);
    }
    // All of these are workgroup-uniform; the integer divisions leave them in
    // vector registers, and the buffer descriptors and offsets built from
    // them must be scalar (else every load becomes a loop over lanes).
    it.tm = __builtin_amdgcn_readfirstlane(tm);
    it.tn = __builtin_amdgcn_readfirstlane(tn);
    it.part = __builtin_amdgcn_readfirstlane(part);
    it.split_tile = __builtin_amdgcn_readfirstlane(split_tile);
    it.kt0 = __builtin_amdgcn_readfirstlane(it.part < 0 ? 0 : it.part * (nk / g.split_parts));
    it.kt1 = __builtin_amdgcn_readfirstlane(it.part < 0 ? nk : it.kt0 + nk / g.split_parts);
    it.m0 = (int64_t)it.tm * BM;
    it.n0 = (int64_t)it.tn * BN;
    const int rows_a = (int)(g.m - it.m0 < BM ? g.m - it.m0 : BM);
    const int rows_b = (int)(g.n - it.n0 < BN ? g.n - it.n0 : BN);
    // Stored across K: the buffer starts at the tile's first column and runs
    // to the end of the operand (columns past m but below ld read other
    // columns, which only reach rows of C that are not stored; lanes past ld
    // read 0).
    it.ra = TA
        ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(g.a_codes + it.m0 * 2), 0,
                                            (int)(g.K * g.a_ldb - it.m0 * 2), kBufferFlags)
        : Chunked
        ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(g.a_codes + it.m0 * RBK), 0,
                                            (int)((nk * g.m - it.m0) * RBK), kBufferFlags)
        : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(g.a_codes + it.m0 * Kb), 0,
                                            (int)(rows_a * Kb), kBufferFlags);
    it.rb = TB
        ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(g.b_codes + it.n0 * 2), 0,
                                            (int)(g.K * g.b_ldb - it.n0 * 2), kBufferFlags)
        : Chunked
        ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(g.b_codes + it.n0 * RBK), 0,
                                            (int)((nk * g.n - it.n0) * RBK), kBufferFlags)
        : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(g.b_codes + it.n0 * Kb), 0,
                                            (int)(rows_b * Kb), kBufferFlags);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = row0 + 16 * j;
      if (Chunked) {
        it.voffa[j] = r < rows_a ? r * RBK + chunk * 16 : kPastEnd;
        it.voffb[j] = r < rows_b ? r * RBK + chunk * 16 : kPastEnd;
      } else {
        it.voffa[j] = TA ? tr_voff(j, g.a_ldb, it.m0) : r * (int)Kb + chunk * 16;
        it.voffb[j] = TB ? tr_voff(j, g.b_ldb, it.n0) : r * (int)Kb + chunk * 16;
      }
    }
    it.soff = sc_a ? (srow < rows_a ? (int)((it.m0 + srow) * 4) : kPastEnd)
                   : (srow < rows_b ? (int)((it.n0 + srow) * 4) : kPastEnd);
    return it;
  };

  auto issue = [&](const RingItem& it, auto S, int kt) {
    constexpr int slot = decltype(S)::value;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          it.ra, (lds_void*)&ring_slot<slot>().a[1024 * (2 * wave + j)], 16, it.voffa[j], kt * stage_a, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          it.rb, (lds_void*)&ring_slot<slot>().b[1024 * (2 * wave + j)], 16, it.voffb[j], kt * stage_b, 0, 0);
    }
    if constexpr (!Bf16) {
      if (sc_a)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)&ring_slot<slot>().sa[256 * (wave & 3)],
                                                 4, it.soff, kt * sstage, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)&ring_slot<slot>().sb[256 * (wave & 3)],
                                                 4, it.soff, kt * sstage, 0, 0);
    }
  };
  // Ring load q (0 .. kLoads - 1) of this wave's share of a stage: A rows
  // j = q / 2 (q even), B rows j (q odd), then the scales.
  auto issue_one = [&](const RingItem& it, auto S, auto Q, int kt) {
    constexpr int slot = decltype(S)::value;
    constexpr int q = decltype(Q)::value;
    if constexpr (q < 4) {
      constexpr int j = q >> 1;
      if constexpr ((q & 1) == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            it.ra, (lds_void*)&ring_slot<slot>().a[1024 * (2 * wave + j)], 16, it.voffa[j], kt * stage_a, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            it.rb, (lds_void*)&ring_slot<slot>().b[1024 * (2 * wave + j)], 16, it.voffb[j], kt * stage_b, 0, 0);
    } else if constexpr (!Bf16) {
      if (sc_a)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)&ring_slot<slot>().sa[256 * (wave & 3)],
                                                 4, it.soff, kt * sstage, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)&ring_slot<slot>().sb[256 * (wave & 3)],
                                                 4, it.soff, kt * sstage, 0, 0);
    }
  };
  // A tile's first stages: kt0 .. kt0+2 whole and the first kLoads - 2
  // loads of kt0+3 (its stage kt0 issues the rest).
  constexpr int kFirstLoads = 4 * kLoads - 2;
  auto issue_first = [&](const RingItem& it) {
    issue(it, std::integral_constant<int, 0>{}, it.kt0);
    issue(it, std::integral_constant<int, 1>{}, it.kt0 + 1);
    issue(it, std::integral_constant<int, 2>{}, it.kt0 + 2);
    static_for<kLoads - 2>([&](auto Q) { issue_one(it, std::integral_constant<int, 3>{}, Q, it.kt0 + 3); });
  };

  v16f acc[R8_FM][R8_FN];

  const int lrow = lane & 31, khalf = lane >> 5;
  const int lswz = ring_swz(lrow);
  const int fa_base = (wm * R8_WM + lrow) * RBK, fb_base = (wn * R8_WN + lrow) * RBK;
  // A stage's scale word of a row holds its four block scales in the order
  // 0, 2, 1, 3: half h of the wave reads the 16 bits at byte 2 h, which hold
  // its K-step 0 and K-step 1 scales in bytes 0 and 1 (the MFMA's op_sel).
  const int sa_off = (wm * R8_WM + lrow) * 4 + 2 * khalf, sb_off = (wn * R8_WN + lrow) * 4 + 2 * khalf;

  // Operands stored across K: per-lane fragment offsets in a slot (K-step 0,
  // read r = 0) of the MFMA blocks i (A) and j (B).
  const int tL = lane & 15, tG = lane >> 4;
  const int th = (tL >> 2) + 4 * (tG >> 1);
  const int tbase = (8 * (tG >> 1) + (tL >> 2)) * 512 + 16 * (2 * (tG & 1) + ((tL & 3) >> 1)) +
                    8 * (tL & 1);
  int toff_a[R8_FM], toff_b[R8_FN];
#pragma unroll
  for (int i = 0; i < R8_FM; ++i) toff_a[i] = tbase + 64 * ((4 * wm + i) ^ th);
#pragma unroll
  for (int j = 0; j < R8_FN; ++j) toff_b[j] = tbase + 64 * ((2 * wn + j) ^ th);
  auto tr_frag = [](const uint8_t* p) {
    typedef __attribute__((address_space(3))) v4s16 lds_v4s16;
    const v4s16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16*)(p));
    const v4s16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16*)(p + 2048));
    const v2i l = __builtin_bit_cast(v2i, lo), h = __builtin_bit_cast(v2i, hi);
    return v4i{l[0], l[1], h[0], h[1]};
  };

  // Fragments of one K-step (16 bytes each) with the stage's scale words.
  struct Frags {
    v4i a[R8_FM], b[R8_FN];
    int sa[R8_FM], sb[R8_FN];
  };
  // Keeps a fragment set live up to this point, so that the other set (read
  // meanwhile) gets registers of its own: a read into a register that an
  // in-flight MFMA still reads would have to wait for that MFMA.
  auto keep = [](const Frags& f) {
    if constexpr (Bf16)
      asm volatile("" ::"v"(f.a[0]), "v"(f.a[1]), "v"(f.a[2]), "v"(f.a[3]), "v"(f.b[0]), "v"(f.b[1]));
    else
      asm volatile("" ::"v"(f.a[0]), "v"(f.a[1]), "v"(f.a[2]), "v"(f.a[3]), "v"(f.b[0]), "v"(f.b[1]),
                   "v"(f.sa[0]), "v"(f.sa[1]), "v"(f.sa[2]), "v"(f.sa[3]), "v"(f.sb[0]), "v"(f.sb[1]));
  };
  auto read_frags = [&](auto S, auto KS, Frags& f) {
    constexpr int slot = decltype(S)::value;
    constexpr int ks = decltype(KS)::value;
    const int sw = ((2 * ks + khalf) ^ lswz) << 4;
    if constexpr (!Bf16 && ks == 0) {
#pragma unroll
      for (int i = 0; i < R8_FM; ++i)
        f.sa[i] = *reinterpret_cast<const uint16_t*>(&ring_slot<slot>().sa[sa_off + 128 * i]);
#pragma unroll
      for (int j = 0; j < R8_FN; ++j)
        f.sb[j] = *reinterpret_cast<const uint16_t*>(&ring_slot<slot>().sb[sb_off + 128 * j]);
    }
#pragma unroll
    for (int i = 0; i < R8_FM; ++i) {
      if constexpr (TA)
        f.a[i] = tr_frag(&ring_slot<slot>().a[toff_a[i] + 8192 * ks]);
      else
        f.a[i] = *reinterpret_cast<const v4i*>(&ring_slot<slot>().a[fa_base + sw + 2048 * i]);
    }
#pragma unroll
    for (int j = 0; j < R8_FN; ++j) {
      if constexpr (TB)
        f.b[j] = tr_frag(&ring_slot<slot>().b[toff_b[j] + 8192 * ks]);
      else
        f.b[j] = *reinterpret_cast<const v4i*>(&ring_slot<slot>().b[fb_base + sw + 2048 * j]);
    }
  };
  // 8 MFMAs of K-step ks: scale byte ks of the 16 bits read.
  auto mma = [&](const Frags& f, auto KS) {
    constexpr int kSel = decltype(KS)::value;
    static_for<R8_FM>([&](auto I) {
      static_for<R8_FN>([&](auto J) {
        const v4i fb = f.b[J], fa = f.a[I];
        if constexpr (Bf16)
          acc[I][J] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(v8bf, fb), __builtin_bit_cast(v8bf, fa), acc[I][J], 0, 0, 0);
        else
          acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              v8i{fb[0], fb[1], fb[2], fb[3], 0, 0, 0, 0}, v8i{fa[0], fa[1], fa[2], fa[3], 0, 0, 0, 0},
              acc[I][J], 4, 4, kSel, f.sb[J], kSel, f.sa[I]);
      });
    });
  };

  // Stage kt (its K-step 0 fragments in x): read K-step 1 into y during
  // K-step 0's MFMAs; wait until only this wave's loads of stages kt+2,
  // kt+3 are in flight and sync, publishing stage kt+1 and freeing slot kt;
  // refill it with stage kt+4 (past kt1: a re-load of the last stage no one
  // reads) and read stage kt+1's K-step 0 into x during K-step 1's MFMAs.
  // A stage's ring loads are spread over the 16 MFMAs between two syncs:
  // the first kLoads - 2 among K-step 1's MFMAs of stage kt, the last two
  // among K-step 0's of stage kt+1 (the slot is free since the sync, and
  // the next sync still counts them as in flight). Issued back to back,
  // the 40 loads of a workgroup stall the waves behind them on the vector
  // memory path while the matrix cores wait.
  constexpr int kEarly = kLoads - 2;      // ring loads of a stage issued right after the sync
  auto stage = [&](const RingItem& it, auto S, Frags& x, Frags& y, int kt) {
    constexpr int slot = decltype(S)::value;
    read_frags(std::integral_constant<int, slot>{}, std::integral_constant<int, 1>{}, y);
    if constexpr (!Bf16) {
      // K-step 1 uses the scale registers read with K-step 0 (x's are
      // replaced by the next stage's before y's MFMAs run).
#pragma unroll
      for (int i = 0; i < R8_FM; ++i) y.sa[i] = x.sa[i];
#pragma unroll
      for (int j = 0; j < R8_FN; ++j) y.sb[j] = x.sb[j];
    }
    {
      // The last two loads of stage kt+3 (slot (slot + 3) % 4).
      const int kt3 = kt + 3 < it.kt1 ? kt + 3 : it.kt1 - 1;
      issue_one(it, std::integral_constant<int, (slot + 3) % kRingSlots>{},
                std::integral_constant<int, kEarly>{}, kt3);
      issue_one(it, std::integral_constant<int, (slot + 3) % kRingSlots>{},
                std::integral_constant<int, kEarly + 1>{}, kt3);
    }
    mma(x, std::integral_constant<int, 0>{});
    // 8 MFMAs with the 2 loads and kDs1 fragment reads between them.
    static_for<6>([&](auto S) {
      constexpr int s = decltype(S)::value;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      if constexpr (s == 1 || s == 4) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // VMEM
      __builtin_amdgcn_sched_group_barrier(0x100, kDs1 / 6 + (s < kDs1 % 6 ? 1 : 0), 0);   // DS read
    });
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    keep(x);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * kLoads, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    {
      const int kt4 = kt + 4 < it.kt1 ? kt + 4 : it.kt1 - 1;
      static_for<kEarly>([&](auto Q) { issue_one(it, std::integral_constant<int, slot>{}, Q, kt4); });
    }
    read_frags(std::integral_constant<int, (slot + 1) % kRingSlots>{}, std::integral_constant<int, 0>{}, x);
    mma(y, std::integral_constant<int, 1>{});
    // 8 MFMAs with the kEarly loads and kDs fragment reads between them.
    static_for<6>([&](auto S) {
      constexpr int s = decltype(S)::value;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      if constexpr (s % 2 == 0 && s / 2 < kEarly) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // VMEM
      __builtin_amdgcn_sched_group_barrier(0x100, kDs / 6 + (s < kDs % 6 ? 1 : 0), 0);   // DS read
    });
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    keep(y);
  };

  // The outer outlier product's items (FP4 kernel with oe_items > 0): each
  // workgroup b < oe_items runs item b once, before its tile round
  // (b / oe_tiles_w) % 4 (or after its last one): at any time about a
  // quarter of the items stream the bf16 operand from memory while the other
  // workgroups keep the matrix cores busy, and the items that run together
  // cover whole rows of it (all wide blocks of one K-part). Work w of the
  // sequence: >= 0 a tile item, kOeWork the outlier item, kNoWork none.
  constexpr int kNoWork = -1, kOeWork = -2;
  const bool has_oe = !Bf16 && bid < g.oe_items;
  const int my_rounds = items > bid ? (items - bid + G - 1) / G : 0;
  const int oe_slot = has_oe ? (bid / g.oe_tiles_w) & 3 : 0;
  const int oe_at = has_oe ? (oe_slot < my_rounds ? oe_slot : my_rounds) : -1;
  auto work_at = [&](int q) {
    if (has_oe) {
      if (q == oe_at) return kOeWork;
      if (q > oe_at) --q;
    }
    return item_of(q);
  };
  // Outlier item e = bid: 256-wide block e % oe_tiles_w of the operand
  // stored across K (A-side of the slot, read as in TA mode), K-part
  // e / oe_tiles_w; its lines ([k][K] bf16 rows) in the B-side rows 0 .. 63.
  // The outlier item's per-lane offsets are computed inside its branch from
  // a lane id the compiler cannot see through: hoisted out of the work loop
  // they would stay live across the tiles' K loop, which has no registers to
  // spare.
  auto opaque_lane = [&]() {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  auto setup_oe = [&]() {
    RingItem it;
    const int ol = opaque_lane();
    const int orow0 = 32 * wave + (ol >> 2);
    const int ochunk = (ol & 3) ^ ring_swz(orow0);
    auto otr_voff = [&](int j, int64_t ldb, int64_t c0) {
      const int k = 2 * (2 * wave + j) + (ol >> 5);
      const int h = (k & 3) | (((k >> 3) & 1) << 2);
      const int c = (ol & 31) ^ (4 * h);
      return 8 * (int64_t)c < ldb / 2 - c0 ? k * (int)ldb + 16 * c : kPastEnd;
    };
    const int wt = __builtin_amdgcn_readfirstlane(bid % g.oe_tiles_w);
    const int sp = __builtin_amdgcn_readfirstlane(bid / g.oe_tiles_w);
    it.tm = wt; it.tn = 0; it.part = sp; it.split_tile = 0;
    it.kt0 = __builtin_amdgcn_readfirstlane(sp * g.oe_kst);
    it.kt1 = __builtin_amdgcn_readfirstlane(it.kt0 + g.oe_kst);
    it.m0 = (int64_t)wt * BM;
    it.n0 = 0;
    it.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(g.oe_wide + it.m0 * 2), 0,
                                              (int)(g.K * g.oe_wide_ldb - it.m0 * 2), kBufferFlags);
    it.rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(g.oe_lines), 0,
                                              (int)(g.oe_k * g.K * 2), kBufferFlags);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = orow0 + 16 * j;
      it.voffa[j] = otr_voff(j, g.oe_wide_ldb, it.m0);
      it.voffb[j] = r < g.oe_k ? r * (int)(2 * g.K) + ochunk * 16 : kPastEnd;
    }
    it.soff = kPastEnd;
    return it;
  };
  // Waves 0 and 1 also copy the stage's 64 line rows (4 loads per stage),
  // the others only their share of the wide operand (2 loads).
  auto issue_oe = [&](const RingItem& it, auto S, int kt) {
    constexpr int slot = decltype(S)::value;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          it.ra, (lds_void*)&ring_slot<slot>().a[1024 * (2 * wave + j)], 16, it.voffa[j],
          kt * 32 * (int)g.oe_wide_ldb, 0, 0);
    if (wave < 2) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            it.rb, (lds_void*)&ring_slot<slot>().b[1024 * (2 * wave + j)], 16, it.voffb[j], kt * RBK, 0, 0);
    }
  };
  // Waits until only this wave's loads of the `later` stages after the one
  // wanted are in flight (4 or 2 loads per stage, as above).
  auto oe_wait = [&](auto Later) {
    constexpr int later = decltype(Later)::value;
    if (wave < 2) __builtin_amdgcn_s_waitcnt(waitcnt_imm(4 * later, 0));
    else __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * later, 0));
  };
  auto issue_first4_oe = [&](const RingItem& it) {
    issue_oe(it, std::integral_constant<int, 0>{}, it.kt0);
    issue_oe(it, std::integral_constant<int, 1>{}, it.kt0 + 1);
    issue_oe(it, std::integral_constant<int, 2>{}, it.kt0 + 2);
    issue_oe(it, std::integral_constant<int, 3>{}, it.kt0 + 3);
  };
  auto issue_work = [&](int w) {
    if (w == kOeWork) issue_first4_oe(setup_oe());
    else if (w >= 0) issue_first(setup(w));
  };
  // One bf16 stage (32 K-elements, two 16-deep steps) of the outlier item:
  // wave w's 32 wide rows (block w of the slot, transposing reads) against
  // the 64 lines; then, once every wave has its loads of the next stage and
  // no wave reads this slot any more, the slot is refilled 4 stages ahead.
  // Fragment offsets of the outlier item (block `wave` of the wide operand,
  // read transposed; rows 0 .. 63 of the lines), from the opaque lane id.
  struct OeOff {
    int w, n;
    int swz;
  };
  auto oe_offsets = [&]() {
    const int ol = opaque_lane();
    const int oL = ol & 15, oG = ol >> 4;
    const int oth = (oL >> 2) + 4 * (oG >> 1);
    const int obase = (8 * (oG >> 1) + (oL >> 2)) * 512 + 16 * (2 * (oG & 1) + ((oL & 3) >> 1)) +
                      8 * (oL & 1);
    const int orow = ol & 31;
    return OeOff{obase + 64 * (wave ^ oth), orow * RBK, ring_swz(orow) | ((ol >> 5) << 8)};
  };
  auto oe_stage = [&](const RingItem& it, auto S, v16f (&oacc)[2], const OeOff& o, int kt) {
    constexpr int slot = decltype(S)::value;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const v4i fw = tr_frag(&ring_slot<slot>().a[o.w + 8192 * ks]);
      const int sw = ((2 * ks + (o.swz >> 8)) ^ (o.swz & 3)) << 4;
      const v4i fn0 = *reinterpret_cast<const v4i*>(&ring_slot<slot>().b[o.n + sw]);
      const v4i fn1 = *reinterpret_cast<const v4i*>(&ring_slot<slot>().b[o.n + sw + 2048]);
      oacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, fn0),
                                                        __builtin_bit_cast(v8bf, fw), oacc[0], 0, 0, 0);
      oacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, fn1),
                                                        __builtin_bit_cast(v8bf, fw), oacc[1], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    oe_wait(std::integral_constant<int, 2>{});
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_oe(it, std::integral_constant<int, slot>{}, kt + 4 < it.kt1 ? kt + 4 : it.kt1 - 1);
  };

  int work = work_at(0);
  if (work == kNoWork) return;
  issue_work(work);
  for (int q = 0;; ++q) {
    // Only the work index is carried over: the item's descriptors are built
    // again here from scalars (carried through the loop they would end up in
    // vector registers).
    work = __builtin_amdgcn_readfirstlane(work);
    if constexpr (!Bf16) {
      if (work == kOeWork) {
        const RingItem cur = setup_oe();
        v16f oacc[2];
#pragma unroll
        for (int v = 0; v < 16; ++v) { oacc[0][v] = 0.0f; oacc[1][v] = 0.0f; }
        oe_wait(std::integral_constant<int, 3>{});
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const OeOff o = oe_offsets();
        for (int kt = cur.kt0; kt < cur.kt1; kt += kRingSlots) {
          oe_stage(cur, std::integral_constant<int, 0>{}, oacc, o, kt);
          oe_stage(cur, std::integral_constant<int, 1>{}, oacc, o, kt + 1);
          oe_stage(cur, std::integral_constant<int, 2>{}, oacc, o, kt + 2);
          oe_stage(cur, std::integral_constant<int, 3>{}, oacc, o, kt + 3);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        __syncthreads();
        const int next = work_at(q + 1);
        issue_work(next);
        // Partial sums of K-part cur.part: lane l holds wide row w (column
        // l % 32 of the MFMA result), register v line 32 j + acc_row(v, l).
        const int ol = opaque_lane();
        const int64_t w = cur.m0 + 32 * wave + (ol & 31);
        if (w < g.oe_wide_n) {
          const bool right = g.oe_mode == ADAHOP_ROUTE_OE_RIGHT;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int p = 32 * j + acc_row(v, ol);
              if (p >= g.oe_k) continue;
              const int64_t at = right ? ((int64_t)cur.part * g.oe_wide_n + w) * g.oe_k + p
                                       : ((int64_t)cur.part * g.oe_k + p) * g.oe_wide_n + w;
              g.oe_part[at] = oacc[j][v];
            }
          }
        }
        if (next == kNoWork) break;
        work = next;
        continue;
      }
    }
    const int item = work;
    const RingItem cur = setup(item);
    static_for<R8_FM>([&](auto I) {
      static_for<R8_FN>([&](auto J) {
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[I][J][v] = 0.0f;
      });
    });
    Frags fx, fy;
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(kFirstLoads - kLoads, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, fx);
    for (int kt = cur.kt0; kt < cur.kt1; kt += kRingSlots) {
      stage(cur, std::integral_constant<int, 0>{}, fx, fy, kt);
      stage(cur, std::integral_constant<int, 1>{}, fx, fy, kt + 1);
      stage(cur, std::integral_constant<int, 2>{}, fx, fy, kt + 2);
      stage(cur, std::integral_constant<int, 3>{}, fx, fy, kt + 3);
    }

    // Every wave's last reads and loads of the ring are done before it is
    // refilled with the next item's first stages (or handed on).
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __syncthreads();
    const int next = work_at(q + 1);
    issue_work(next);

    // The inner-extraction term goes into a whole tile or part 0 of a split
    // one. A part of a split tile then goes out through the same store code,
    // as a plain fp32 256 x 256 matrix (one code path keeps the accumulators
    // in registers); the fixup kernel adds the outer-extraction term.
    if (cur.part <= 0) gemm_inner_term<R8_FM, R8_FN, R8_WM, R8_WN, 4>(g, acc, cur.m0, cur.n0);
    GemmArgs ge = g;
    int64_t em0 = cur.m0, en0 = cur.n0;
    if (cur.part >= 0) {
      ge.C = g.split_ws + ((size_t)cur.split_tile * g.split_parts + cur.part) * (size_t)(BM * BN);
      ge.ldc = BN; ge.m = BM; ge.n = BN; ge.out_f32 = 1; ge.vec_ok = 1; ge.oe_mode = 0;
      em0 = 0; en0 = 0;
    }
    gemm_store<R8_FM, R8_FN, R8_WM, R8_WN, 4, kRing8Threads>(ge, acc, em0, en0, g_ring_pos);
    if (next == kNoWork) break;
    // No wait for the epilogue's stores here: the next item's waits count
    // only ring loads issued after the ones they wait for, and loads return
    // in order, so stores (or epilogue loads) still in flight can only make
    // those waits stricter, never let one pass early. The stores drain
    // while the next item starts (a wait here cost 1-9 % of the GEMM on
    // short-K shapes, where every CU stores its tile at the same moment).
    work = next;
  }
}

// Adds the parts of the split tiles in part order, adds the outer-extraction
// term (OE_LEFT rows / OE_RIGHT columns) and writes C with one rounding, as
// the main kernel's epilogue does for a whole tile. Workgroup b takes rows
// 16 (b % 16) .. +15 of split tile b / 16; thread t columns 4 (t % 64) .. +3
// of rows t / 64 + 4 i, so every read of a part is a 1 KB row run.
constexpr int kFixThreads = 256, kFixRows = 16;
__global__ void __launch_bounds__(kFixThreads) gemm_split_fixup_kernel(GemmArgs g) {
  __shared__ int s_pos[BM > BN ? BM : BN];
  const int tile = blockIdx.x / (BM / kFixRows), band = blockIdx.x % (BM / kFixRows);
  int tm, tn;
  tile_at(g.split_full + tile, g.tiles_m, g.tiles_n, &tm, &tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int tid = threadIdx.x;
  const bool oe_rows = g.oe_mode == ADAHOP_ROUTE_OE_LEFT;
  const bool oe_cols = g.oe_mode == ADAHOP_ROUTE_OE_RIGHT;
  bool any_oe = false;
  if (oe_rows || oe_cols) {
    const int64_t lo_v = oe_rows ? m0 : n0;
    const int span = oe_rows ? BM : BN;
    const int lo = lower_bound_i32(g.oe_idx, g.oe_k, lo_v);
    const int hi = lower_bound_i32(g.oe_idx, g.oe_k, lo_v + span);
    any_oe = hi > lo;
    if (any_oe) {
      for (int q = tid; q < span; q += kFixThreads) s_pos[q] = -1;
      __syncthreads();
      for (int p = lo + tid; p < hi; p += kFixThreads) s_pos[g.oe_idx[p] - lo_v] = p;
      __syncthreads();
    }
  }
  const int lc = 4 * (tid % 64);
  const int64_t col = n0 + lc;
  const float* part0 = g.split_ws + (size_t)tile * g.split_parts * (size_t)(BM * BN);
#pragma unroll
  for (int i = 0; i < kFixRows / 4; ++i) {
    const int lr = band * kFixRows + tid / 64 + 4 * i;
    const int64_t row = m0 + lr;
    if (row >= g.m || col >= g.n) continue;
    float4 a = *reinterpret_cast<const float4*>(part0 + lr * BN + lc);
    for (int p = 1; p < g.split_parts; ++p) {
      const float4 b = *reinterpret_cast<const float4*>(part0 + (size_t)p * (BM * BN) + lr * BN + lc);
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    float v[4] = {a.x, a.y, a.z, a.w};
    if (any_oe && g.oe_res) {
      // The outlier product was computed in the main kernel: keep the
      // residual of the extracted lines for oe_scatter_kernel.
      if (oe_rows) {
        const int prow = s_pos[lr];
        if (prow >= 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < g.n) g.oe_res[(int64_t)prow * g.n + col + e] = v[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = s_pos[lc + e];
          if (p >= 0) g.oe_res[row * g.oe_k + p] = v[e];
        }
      }
    } else if (any_oe) {
      if (oe_rows) {
        const int prow = s_pos[lr];
        if (prow >= 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < g.n) v[e] += g.oe_p[(int64_t)prow * g.n + col + e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = s_pos[lc + e];
          if (p >= 0) v[e] += g.oe_p[row * g.oe_k + p];
        }
      }
    }
    if (col + 4 <= g.n && g.vec_ok) {
      if (g.out_f32) {
        *reinterpret_cast<float4*>(static_cast<float*>(g.C) + row * g.ldc + col) =
            make_float4(v[0], v[1], v[2], v[3]);
      } else {
        const uint32_t lo = f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.C) + row * g.ldc + col) = make_uint2(lo, hi);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (col + e >= g.n) continue;
        if (g.out_f32)
          static_cast<float*>(g.C)[row * g.ldc + col + e] = v[e];
        else
          static_cast<uint16_t*>(g.C)[row * g.ldc + col + e] = f32_to_bf16_rne(v[e]);
      }
    }
  }
}

// The outer outlier product computed inside the main kernel, scattered into
// C: for every wide index w and line p, C at (w, idx[p]) (OE_RIGHT) or
// (idx[p], w) (OE_LEFT) becomes the extracted line's fp32 residual, kept by
// the tile epilogue or the fixup, plus the partial sums added in part order,
// rounded once. Thread t takes (w, p) in the partials' own order, so the
// reads of every part are coalesced; it loads eight parts at a time before
// adding them in order, so the loads are in flight together.
__global__ void __launch_bounds__(256) oe_scatter_kernel(GemmArgs g, int parts) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t count = g.oe_wide_n * g.oe_k;
  if (t >= count) return;
  const float res = g.oe_res[t];
  float sum = g.oe_part[t];
  int s = 1;
  for (; s + 8 <= parts; s += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = g.oe_part[(int64_t)(s + j) * count + t];
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += v[j];
  }
  for (; s < parts; ++s) sum += g.oe_part[(int64_t)s * count + t];
  const float v = res + sum;
  const bool right = g.oe_mode == ADAHOP_ROUTE_OE_RIGHT;
  const int64_t w = right ? t / g.oe_k : t % g.oe_wide_n;
  const int p = (int)(right ? t % g.oe_k : t / g.oe_wide_n);
  const int64_t row = right ? w : g.oe_idx[p];
  const int64_t col = right ? g.oe_idx[p] : w;
  if (g.out_f32) static_cast<float*>(g.C)[row * g.ldc + col] = v;
  else static_cast<uint16_t*>(g.C)[row * g.ldc + col] = f32_to_bf16_rne(v);
}

// ---------------------------------------------------------------------------
// bf16 product on matrix cores: P[x][y] = sum_t X(x,t) * Y(y,t), split over K.
// Memory-bound (it streams the whole bf16 operand). A workgroup computes a
// 128 x 64 tile (wave w: rows 32 w .. +31, both 32-column halves) with
// v_mfma_f32_32x32x16_bf16 over 64-element K stages, double buffered in LDS
// and prefetched one stage ahead in registers. Global loads are 16 bytes per
// lane along each view's contiguous direction and land in LDS in that same
// order (OeTile); an x-contiguous view is transposed by the fragment reads.
// ---------------------------------------------------------------------------
constexpr int OX = 128, OY = 64, OK = 64, OPAD = 72, kOeThreads = 256;

struct OeArgs {
  const uint16_t* x; int64_t xld;
  const uint16_t* y; int64_t yld;
  int64_t nx, ny, K, kchunk;
  float* partials;                 // [splits][nx][ny], or nullptr
  void* C; int64_t ldc; int out_f32;   // direct output when partials == nullptr
};

// LDS tile of a view for one K stage: a t-contiguous (Inner) view is stored
// as [R][OPAD] rows of t; an x-contiguous view keeps its memory order as
// [OK][R + 4] rows of x. The x-major pitch (R + 4 elements: 264 or 136 bytes)
// puts rows t and t + 8 -- read by the two half-waves of one fragment read --
// 64 bytes apart modulo 256, so those reads are free of bank conflicts.
template <int R, bool Inner>
struct OeTile {
  static constexpr int kElems = Inner ? R * OPAD : OK * (R + 4);
};

// Loads one [R][OK] tile of a view, starting at (r0, t0), into registers and
// stores it into LDS in the OeTile layout.
template <int R, bool Inner>
struct TileLoader {
  // Each 16-byte chunk: Inner: row r, t-chunk c (8 t); else: t row, x-chunk (8 x).
  static constexpr int kChunks = R * OK / 8;
  static constexpr int kPerThread = kChunks / kOeThreads;
  static constexpr int kXPitch = R + 4;
  uint4 v[kPerThread];
  __device__ __forceinline__ void load(const uint16_t* p, int64_t ld, int64_t r0, int64_t nr,
                                       int64_t t0, int64_t t1) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int e = threadIdx.x + i * kOeThreads;
      int64_t gr, gt;
      if (Inner) { gr = r0 + e / (OK / 8); gt = t0 + (e % (OK / 8)) * 8; }
      else       { gt = t0 + e / (R / 8);  gr = r0 + (e % (R / 8)) * 8; }
      // 8 consecutive elements along the contiguous direction; edges padded with 0.
      uint4 q = make_uint4(0, 0, 0, 0);
      if (Inner) {
        if (gr < nr) {
          if (gt + 8 <= t1 && ((ld | gt) & 7) == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
            q = *reinterpret_cast<const uint4*>(p + gr * ld + gt);
          } else {
            uint16_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) h[j] = gt + j < t1 ? p[gr * ld + gt + j] : 0;
            q = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
          }
        }
      } else {
        if (gt < t1) {
          if (gr + 8 <= nr && ((ld | gr) & 7) == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
            q = *reinterpret_cast<const uint4*>(p + gt * ld + gr);
          } else {
            uint16_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) h[j] = gr + j < nr ? p[gt * ld + gr + j] : 0;
            q = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
          }
        }
      }
      v[i] = q;
    }
  }
  __device__ __forceinline__ void store(uint16_t* s) const {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int e = threadIdx.x + i * kOeThreads;
      if (Inner) {
        const int r = e / (OK / 8), c = (e % (OK / 8)) * 8;
        *reinterpret_cast<uint4*>(&s[r * OPAD + c]) = v[i];
      } else {
        const int t = e / (R / 8), r = (e % (R / 8)) * 8;
        uint2* d = reinterpret_cast<uint2*>(&s[t * kXPitch + r]);   // 8-byte aligned
        d[0] = make_uint2(v[i].x, v[i].y);
        d[1] = make_uint2(v[i].z, v[i].w);
      }
    }
  }
  // The MFMA fragment of row r (of this tile) for t = t0 .. t0 + 7.
  __device__ __forceinline__ static v8bf frag(const uint16_t* s, int r, int t0) {
    uint4 q;
    if (Inner) {
      q = *reinterpret_cast<const uint4*>(&s[r * OPAD + t0]);
    } else {
      uint32_t h[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = s[(t0 + j) * kXPitch + r];
      q = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    }
    return __builtin_bit_cast(v8bf, q);
  }
};

template <bool XIn, bool YIn>
__global__ void __launch_bounds__(kOeThreads) oe_product_kernel(OeArgs g) {
  using LX = TileLoader<OX, XIn>;
  using LY = TileLoader<OY, YIn>;
  __shared__ __attribute__((aligned(16))) uint16_t sx[2][OeTile<OX, XIn>::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t sy[2][OeTile<OY, YIn>::kElems];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t x0 = (int64_t)blockIdx.x * OX, y0 = (int64_t)blockIdx.y * OY;
  const int64_t tb = (int64_t)blockIdx.z * g.kchunk;
  const int64_t te = (tb + g.kchunk < g.K) ? tb + g.kchunk : g.K;
  v16f acc0, acc1;
#pragma unroll
  for (int v = 0; v < 16; ++v) { acc0[v] = 0.0f; acc1[v] = 0.0f; }
  LX lx;
  LY ly;
  const int nst = (int)((te - tb + OK - 1) / OK);
  if (nst > 0) {
    lx.load(g.x, g.xld, x0, g.nx, tb, te);
    ly.load(g.y, g.yld, y0, g.ny, tb, te);
    lx.store(sx[0]);
    ly.store(sy[0]);
  }
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) {
      lx.load(g.x, g.xld, x0, g.nx, tb + (int64_t)(st + 1) * OK, te);
      ly.load(g.y, g.yld, y0, g.ny, tb + (int64_t)(st + 1) * OK, te);
    }
#pragma unroll
    for (int ks = 0; ks < OK; ks += 16) {
      const int off = ks + 8 * (lane >> 5);
      const v8bf fa = LX::frag(sx[buf], wave * 32 + (lane & 31), off);
      const v8bf fb0 = LY::frag(sy[buf], lane & 31, off);
      const v8bf fb1 = LY::frag(sy[buf], 32 + (lane & 31), off);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb1, acc1, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (st + 1 < nst) {
      lx.store(sx[buf ^ 1]);
      ly.store(sy[buf ^ 1]);
    }
    __syncthreads();
  }
  // acc_h: rows x0 + 32 wave + acc_row(v), column y0 + 32 h + lane % 32
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t col = y0 + 32 * h + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = x0 + wave * 32 + acc_row(v, lane);
      if (row >= g.nx || col >= g.ny) continue;
      const float val = h == 0 ? acc0[v] : acc1[v];
      if (g.partials) {
        g.partials[(int64_t)blockIdx.z * g.nx * g.ny + row * g.ny + col] = val;
      } else if (g.out_f32) {
        static_cast<float*>(g.C)[row * g.ldc + col] = val;
      } else {
        static_cast<uint16_t*>(g.C)[row * g.ldc + col] = f32_to_bf16_rne(val);
      }
    }
  }
}

void launch_oe(const OeArgs& a, dim3 grid, bool xin, bool yin, hipStream_t stream) {
  if (xin && yin) oe_product_kernel<true, true><<<grid, dim3(kOeThreads), 0, stream>>>(a);
  else if (xin) oe_product_kernel<true, false><<<grid, dim3(kOeThreads), 0, stream>>>(a);
  else if (yin) oe_product_kernel<false, true><<<grid, dim3(kOeThreads), 0, stream>>>(a);
  else oe_product_kernel<false, false><<<grid, dim3(kOeThreads), 0, stream>>>(a);
}

// P[i] = sum over s of partials[s][i], in the order s = 0, 1, ... Four
// consecutive sums per thread (16-byte loads when count % 4 == 0), eight
// partial arrays' loads in flight before their adds.
__global__ void __launch_bounds__(256) oe_reduce_kernel(const float* __restrict__ partials,
                                                         int splits, int64_t count,
                                                         float* __restrict__ P) {
  const int64_t n4 = (count % 4 == 0) ? count / 4 : 0;
  const float4* p4 = reinterpret_cast<const float4*>(partials);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * 256) {
    float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    int sp = 0;
    for (; sp + 8 <= splits; sp += 8) {
      float4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = p4[(int64_t)(sp + j) * n4 + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) { s.x += v[j].x; s.y += v[j].y; s.z += v[j].z; s.w += v[j].w; }
    }
    for (; sp < splits; ++sp) {
      const float4 v = p4[(int64_t)sp * n4 + i];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    reinterpret_cast<float4*>(P)[i] = s;
  }
  if (n4 > 0) return;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * 256) {
    float s = 0.0f;
    for (int sp = 0; sp < splits; ++sp) s += partials[sp * count + i];
    P[i] = s;
  }
}

}  // namespace

int oe_splits(int64_t nx, int64_t ny, int64_t K) {
  const int64_t tiles = ((nx + OX - 1) / OX) * ((ny + OY - 1) / OY);
  int64_t s = (768 + tiles - 1) / tiles;            // about 3 workgroups per CU
  const int64_t smax = K / 512 > 0 ? K / 512 : 1;   // at least 512 K per split
  if (s > smax) s = smax;
  if (s > 64) s = 64;
  return (int)(s < 1 ? 1 : s);
}

bool oe_product_fits(int64_t nx, int64_t ny) {
  return nx >= 1 && ny >= 1 && (ny + OY - 1) / OY <= 65535 && (nx + OX - 1) / OX <= 0x7FFFFFFF;
}

static int64_t kchunk_for(int64_t K, int splits) {
  int64_t c = (K + splits - 1) / splits;
  return (c + OK - 1) / OK * OK;
}

adahop_status oe_product_launch(Bf16View X, Bf16View Y, int64_t nx, int64_t ny, int64_t K,
                                int splits, float* partials, hipStream_t stream) {
  OeArgs a{X.ptr, X.ld, Y.ptr, Y.ld, nx, ny, K, kchunk_for(K, splits), partials, nullptr, 0, 0};
  const int64_t gy = (ny + OY - 1) / OY;
  if (!oe_product_fits(nx, ny)) return fail(ADAHOP_ERR_UNSUPPORTED, "outlier product: too many columns");
  const dim3 grid((unsigned)((nx + OX - 1) / OX), (unsigned)gy, (unsigned)splits);
  launch_oe(a, grid, X.inner_contiguous != 0, Y.inner_contiguous != 0, stream);
  adahop_status st = check_launch("oe_product");
  if (st != ADAHOP_OK) return st;
  return oe_reduce_launch(partials, splits, nx * ny, stream);
}

adahop_status oe_reduce_launch(float* partials, int splits, int64_t count, hipStream_t stream) {
  float* P = partials + (int64_t)splits * count;
  const int64_t items = count % 4 == 0 ? count / 4 : count;
  const int64_t blocks = (items + 255) / 256 < 1024 ? (items + 255) / 256 : 1024;
  oe_reduce_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(partials, splits, count, P);
  return check_launch("oe_reduce");
}

adahop_status bf16_gemm_launch(Bf16View X, Bf16View Y, int64_t m, int64_t n, int64_t K,
                               void* C, int64_t ldc, int out_f32, hipStream_t stream) {
  const int64_t gx = (m + OX - 1) / OX, gy = (n + OY - 1) / OY;
  if (gx > 0x7FFFFFFF || gy > 65535) return fail(ADAHOP_ERR_UNSUPPORTED, "bf16 gemm: too large");
  OeArgs a{X.ptr, X.ld, Y.ptr, Y.ld, m, n, K, K, nullptr, C, ldc, out_f32};
  launch_oe(a, dim3((unsigned)gx, (unsigned)gy, 1), X.inner_contiguous != 0,
            Y.inner_contiguous != 0, stream);
  return check_launch("bf16_gemm");
}

namespace {

// Stage-major copy of both scale arrays for the main kernel, as 4-byte
// words (the four block scales of one 128-long stage of one row, in the
// order 0, 2, 1, 3): dst[c][r] = src[r][c], c < K/128, through a 64 x 64 LDS
// tile. blockIdx.z picks the operand.
constexpr int kTr = 64;
__global__ void __launch_bounds__(256)
scale_stage_kernel(const uint32_t* __restrict__ sa, int64_t ma, uint32_t* __restrict__ da,
                   const uint32_t* __restrict__ sb, int64_t nb, uint32_t* __restrict__ db,
                   int64_t nst) {
  __shared__ uint32_t tile[kTr][kTr + 1];
  const uint32_t* src = blockIdx.z ? sb : sa;
  uint32_t* dst = blockIdx.z ? db : da;
  const int64_t rows = blockIdx.z ? nb : ma;
  const int64_t r0 = (int64_t)blockIdx.y * kTr, c0 = (int64_t)blockIdx.x * kTr;
  if (r0 >= rows) return;                      // the whole workgroup leaves together
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < kTr; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    if (r < rows && c < nst) tile[i][tx] = src[r * nst + c];
  }
  __syncthreads();
  for (int i = ty; i < kTr; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (r < rows && c < nst) {
      const uint32_t v = tile[tx][i];   // block scales 0, 1, 2, 3 -> stored 0, 2, 1, 3
      dst[c * rows + r] = (v & 0xFF0000FFu) | ((v >> 8) & 0xFF00u) | ((v << 8) & 0xFF0000u);
    }
  }
}

bool ring_shape_ok(int64_t m, int64_t n, int64_t K) {
  const int64_t big = m > n ? m : n;
  return K % 512 == 0 && (m < BM ? m : BM) * (K / 2) < 0x7FFFFFFF &&
         (n < BN ? n : BN) * (K / 2) < 0x7FFFFFFF && big * (K / 32) < 0x7FFFFF00 &&
         (big + kTr - 1) / kTr <= 65535;
}

// Split of the main kernel's last round. One 512-thread workgroup runs per
// CU; when the last round would leave more than half of the CUs idle, its
// tiles are split along K into up to 4 parts (each a multiple of 4 stages
// and at least 16), which a fixup kernel adds. The CU count is the current
// device's, queried once per device (256 on a whole gfx950, and when no
// device can be queried, e.g. for a plan made without a GPU).
constexpr int64_t kDefaultCUs = 256;
int64_t device_cus() {
  static std::mutex mu;
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return kDefaultCUs;
  }
  std::lock_guard<std::mutex> g(mu);
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1) {
      (void)hipGetLastError();
      v = (int)kDefaultCUs;
    }
    cus[dev] = v;
  }
  return cus[dev];
}
struct TailSplit {
  int64_t full, split;   // whole tiles, split tiles
  int parts;
};
// nk: the number of ring stages along K (K / 128 for FP4, K / 32 for bf16).
TailSplit tail_split(int64_t m, int64_t n, int64_t nk) {
  const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  const int64_t cus = device_cus();
  const int64_t rem = tiles % cus;
  int parts = 1;
  if (rem > 0 && 2 * rem <= cus) {
    parts = (int)(cus / rem < 4 ? cus / rem : 4);
    while (parts > 1 && (nk % (4 * parts) != 0 || nk / parts < 16)) --parts;
  }
  if (parts < 2) return {tiles, 0, 1};
  return {tiles - rem, rem, parts};
}

size_t split_ws_bytes(int64_t m, int64_t n, int64_t nk) {
  const TailSplit ts = tail_split(m, n, nk);
  return (size_t)ts.split * (size_t)ts.parts * (size_t)kSplitPartF4 * sizeof(float4);
}

size_t staging_bytes(int64_t m, int64_t n, int64_t K) {
  return align_up((size_t)m * (size_t)(K / 32), kAlign) + align_up((size_t)n * (size_t)(K / 32), kAlign);
}

}  // namespace

bool gemm_mx_fits(int64_t m, int64_t n) {
  return m >= 1 && n >= 1 && ((m + BM - 1) / BM) * ((n + BN - 1) / BN) <= 0x7FFFFFFF;
}

bool gemm_mx_kchunk_ok(int64_t m, int64_t n, int64_t K) {
  const int64_t big = m > n ? m : n;
  return ring_shape_ok(m, n, K) && big * (K / 2) < 0x7FFF0000;   // stage offsets fit 31 bits
}

size_t gemm_mx_scratch_bytes(int64_t m, int64_t n, int64_t K, int layout) {
  if (m < 1 || n < 1 || !ring_shape_ok(m, n, K)) return 0;
  return (layout == ADAHOP_LAYOUT_ROWS ? staging_bytes(m, n, K) : 0) + split_ws_bytes(m, n, K / 128);
}

namespace {
bool ring_applies(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                  const uint8_t* b_scales, int64_t m, int64_t n, int64_t K) {
  const uintptr_t sc_bits = reinterpret_cast<uintptr_t>(a_scales) | reinterpret_cast<uintptr_t>(b_scales);
  const uintptr_t cd_bits = reinterpret_cast<uintptr_t>(a_codes) | reinterpret_cast<uintptr_t>(b_codes);
  return ring_shape_ok(m, n, K) && (sc_bits & 3u) == 0 && (cd_bits & 15u) == 0;
}

adahop_status check_scratch(void* scratch, size_t scratch_bytes, size_t need) {
  if (need == 0) return ADAHOP_OK;
  if (scratch == nullptr || scratch_bytes < need || (reinterpret_cast<uintptr_t>(scratch) & 15u))
    return fail(ADAHOP_ERR_WORKSPACE, "gemm_mx: the main kernel needs " + std::to_string(need) +
                                          " bytes of 16-byte aligned workspace");
  return ADAHOP_OK;
}

uint32_t* staged_b(void* scratch, int64_t m, int64_t K) {
  return static_cast<uint32_t*>(scratch) + align_up((size_t)m * (size_t)(K / 32), kAlign) / 4;
}
}  // namespace

bool gemm_mx_ring_used(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                       const uint8_t* b_scales, int64_t m, int64_t n, int64_t K, int layout) {
  if (layout == ADAHOP_LAYOUT_KCHUNK) return gemm_mx_kchunk_ok(m, n, K);
  return ring_applies(a_codes, a_scales, b_codes, b_scales, m, n, K);
}

int oe_fused_parts(int64_t m, int64_t n, int64_t K, int mode, int32_t k, Bf16View a, Bf16View b,
                   bool check_ptrs) {
  if ((mode != ADAHOP_ROUTE_OE_LEFT && mode != ADAHOP_ROUTE_OE_RIGHT) || k < 1 || k > 64) return 0;
  if (!ring_shape_ok(m, n, K)) return 0;
  const bool right = mode == ADAHOP_ROUTE_OE_RIGHT;
  const Bf16View wide = right ? a : b, lines = right ? b : a;
  const int64_t wide_n = right ? m : n;
  if (wide.inner_contiguous || wide.ld % 8 != 0 || wide.ld < wide_n || K * wide.ld * 2 >= kPastEnd)
    return 0;
  if (!lines.inner_contiguous || lines.ld % 8 != 0 || lines.ld < K || (int64_t)k * lines.ld * 2 >= kPastEnd)
    return 0;
  if (lines.ld != K) return 0;   // the kernel's line rows are K elements apart
  if (check_ptrs && ((reinterpret_cast<uintptr_t>(wide.ptr) | reinterpret_cast<uintptr_t>(lines.ptr)) & 15u))
    return 0;
  // About one item per CU: parts = CUs / wide blocks, each a multiple of 4
  // bf16 stages of 32 and at least 8 of them, at most 64 parts.
  const int64_t tiles_w = (wide_n + BM - 1) / BM, nk = K / 32;
  int64_t parts = device_cus() / tiles_w;
  if (parts > 64) parts = 64;
  while (parts > 1 && (nk % (4 * parts) != 0 || nk / parts < 8)) --parts;
  if (parts < 1 || tiles_w * parts > device_cus()) return 0;
  return (int)parts;
}

size_t oe_fused_bytes(int64_t m, int64_t n, int mode, int32_t k, int parts) {
  const int64_t wide_n = mode == ADAHOP_ROUTE_OE_RIGHT ? m : n;
  return align_up(sizeof(float) * (size_t)(parts + 1) * (size_t)wide_n * (size_t)k, kAlign);
}

adahop_status gemm_mx_stage_scales(const uint8_t* a_codes, const uint8_t* a_scales,
                                   const uint8_t* b_codes, const uint8_t* b_scales, int64_t m,
                                   int64_t n, int64_t K, void* scratch, size_t scratch_bytes,
                                   hipStream_t stream) {
  if (!ring_applies(a_codes, a_scales, b_codes, b_scales, m, n, K)) return ADAHOP_OK;
  const adahop_status st =
      check_scratch(scratch, scratch_bytes, gemm_mx_scratch_bytes(m, n, K, ADAHOP_LAYOUT_ROWS));
  if (st != ADAHOP_OK) return st;
  const int64_t nst = K / 128, big = m > n ? m : n;
  const dim3 tgrid((unsigned)((nst + kTr - 1) / kTr), (unsigned)((big + kTr - 1) / kTr), 2);
  scale_stage_kernel<<<tgrid, dim3(256), 0, stream>>>(
      reinterpret_cast<const uint32_t*>(a_scales), m, static_cast<uint32_t*>(scratch),
      reinterpret_cast<const uint32_t*>(b_scales), n, staged_b(scratch, m, K), nst);
  return check_launch("gemm_mx scale staging");
}

adahop_status gemm_mx_launch(const uint8_t* a_codes, const uint8_t* a_scales,
                             const uint8_t* b_codes, const uint8_t* b_scales, int64_t m,
                             int64_t n, int64_t K, int layout, const OeEpilogue& oe, void* C,
                             int64_t ldc, int out_f32, void* scratch, size_t scratch_bytes,
                             hipStream_t stream, hipEvent_t main_done) {
  const int64_t tiles_m = (m + BM - 1) / BM, tiles_n = (n + BN - 1) / BN;
  if (!gemm_mx_fits(m, n)) return fail(ADAHOP_ERR_UNSUPPORTED, "gemm: too large");
  GemmArgs g{};
  g.a_codes = a_codes; g.a_scales = a_scales; g.b_codes = b_codes; g.b_scales = b_scales;
  g.m = m; g.n = n; g.K = K; g.C = C; g.ldc = ldc; g.out_f32 = out_f32;
  g.tiles_m = (int)tiles_m; g.tiles_n = (int)tiles_n;
  g.oe_mode = oe.mode; g.oe_k = oe.k; g.oe_idx = oe.idx;
  g.oe_p = oe.partials ? oe.partials + (int64_t)oe.splits * (oe.mode == ADAHOP_ROUTE_OE_LEFT ? (int64_t)oe.k * n : m * (int64_t)oe.k) : nullptr;
  // Whole-tile rows take 16-byte stores: 4 fp32 or 8 bf16 values.
  g.vec_ok = (ldc % (out_f32 ? 4 : 8) == 0) && ((reinterpret_cast<uintptr_t>(C) & 15u) == 0);
  g.ia_ptr = oe.a.ptr; g.ia_ld = oe.a.ld; g.ia_inner = oe.a.inner_contiguous;
  g.ib_ptr = oe.b.ptr; g.ib_ld = oe.b.ld; g.ib_inner = oe.b.inner_contiguous;
  const int fused = oe.fused_parts;
  if (fused > 0 && !gemm_mx_ring_used(a_codes, a_scales, b_codes, b_scales, m, n, K, layout))
    return fail(ADAHOP_ERR_UNSUPPORTED, "gemm_mx: the outlier items need the main kernel");
  if (fused > 0) {
    // Outer outlier product as work items of the main kernel, scattered by
    // oe_scatter_kernel after it (and after the fixup of split tiles).
    const bool right = oe.mode == ADAHOP_ROUTE_OE_RIGHT;
    const Bf16View wide = right ? oe.a : oe.b, lines = right ? oe.b : oe.a;
    g.oe_wide_n = right ? m : n;
    g.oe_tiles_w = (int)((g.oe_wide_n + BM - 1) / BM);
    g.oe_items = g.oe_tiles_w * fused;
    g.oe_kst = (int)(K / 32 / fused);
    g.oe_wide = reinterpret_cast<const uint8_t*>(wide.ptr);
    g.oe_wide_ldb = 2 * wide.ld;
    g.oe_lines = reinterpret_cast<const uint8_t*>(lines.ptr);
    g.oe_part = oe.fused_ws;
    g.oe_res = oe.fused_ws + (size_t)fused * (size_t)g.oe_wide_n * (size_t)oe.k;
    g.oe_p = nullptr;
  }
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(kGemmThreads);
  const uintptr_t sc_bits = reinterpret_cast<uintptr_t>(a_scales) | reinterpret_cast<uintptr_t>(b_scales);
  const bool kchunk = layout == ADAHOP_LAYOUT_KCHUNK;
  if (kchunk && (!gemm_mx_kchunk_ok(m, n, K) || !ring_applies(a_codes, a_scales, b_codes, b_scales, m, n, K)))
    return fail(ADAHOP_ERR_UNSUPPORTED, "gemm_mx: K-chunked operands need K % 512 == 0 and aligned buffers");
  if (kchunk || ring_applies(a_codes, a_scales, b_codes, b_scales, m, n, K)) {
    const adahop_status st = check_scratch(scratch, scratch_bytes, gemm_mx_scratch_bytes(m, n, K, layout));
    if (st != ADAHOP_OK) return st;
    if (kchunk) {
      g.a_sst = reinterpret_cast<const uint32_t*>(a_scales);
      g.b_sst = reinterpret_cast<const uint32_t*>(b_scales);
    } else {
      // The scales were reordered into `scratch` by gemm_mx_stage_scales.
      g.a_sst = static_cast<const uint32_t*>(scratch);
      g.b_sst = staged_b(scratch, m, K);
    }
    const TailSplit ts = tail_split(m, n, K / 128);
    g.split_full = (int)ts.full;
    g.split_count = (int)ts.split;
    g.split_parts = ts.parts;
    g.split_ws = ts.split ? reinterpret_cast<float*>(static_cast<char*>(scratch) +
                                                     (kchunk ? 0 : staging_bytes(m, n, K)))
                          : nullptr;
    // Persistent: at most one workgroup per CU, and one per outlier item.
    const int64_t items = ts.full + ts.split * ts.parts, cus = device_cus();
    int64_t wgs = items < cus ? items : cus;
    if (g.oe_items > wgs) wgs = g.oe_items;
    const dim3 rgrid((unsigned)wgs);
    if (kchunk)
      gemm_mx_ring8_kernel<true, false><<<rgrid, dim3(kRing8Threads), 0, stream>>>(g);
    else
      gemm_mx_ring8_kernel<false, false><<<rgrid, dim3(kRing8Threads), 0, stream>>>(g);
    {
      const adahop_status ls = record_main_done(main_done, stream, "gemm_mx");
      if (ls != ADAHOP_OK) return ls;
    }
    if (ts.split) {
      const adahop_status ls = check_launch("gemm_mx");
      if (ls != ADAHOP_OK) return ls;
      gemm_split_fixup_kernel<<<dim3((unsigned)(ts.split * (BM / kFixRows))), dim3(kFixThreads), 0,
                                stream>>>(g);
    }
    if (fused > 0) {
      const adahop_status ls = check_launch("gemm_mx");
      if (ls != ADAHOP_OK) return ls;
      const int64_t count = g.oe_wide_n * oe.k;
      oe_scatter_kernel<<<dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream>>>(g, fused);
    }
  } else {
    if (K % 256 == 0 && (sc_bits & 7u) == 0)
      gemm_mx_kernel<true><<<grid, block, 0, stream>>>(g);
    else
      gemm_mx_kernel<false><<<grid, block, 0, stream>>>(g);
    return record_main_done(main_done, stream, "gemm_mx");
  }
  return check_launch("gemm_mx");
}

adahop_status record_main_done(hipEvent_t main_done, hipStream_t stream, const char* what) {
  const adahop_status ls = check_launch(what);
  if (ls != ADAHOP_OK || main_done == nullptr) return ls;
  const hipError_t e = hipEventRecord(main_done, stream);
  return e == hipSuccess ? ADAHOP_OK
                         : fail(ADAHOP_ERR_HIP, std::string("hipEventRecord: ") + hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// BF16 route on the ring kernel: operands bf16 in rows of K (row stride K),
// ring stages of 32 elements. A bf16 tile row of one workgroup is 2 K bytes,
// so 256 of them must stay below kPastEnd.
// ---------------------------------------------------------------------------
bool bf16_ring_ok(int64_t m, int64_t n, int64_t K) {
  const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  return m >= 1 && n >= 1 && K % 128 == 0 && K > 0 && (int64_t)BM * 2 * K < kPastEnd &&
         tiles <= 0x7FFFFFFF;
}

size_t bf16_ring_scratch_bytes(int64_t m, int64_t n, int64_t K) {
  return bf16_ring_ok(m, n, K) ? split_ws_bytes(m, n, K / 32) : 0;
}

bool bf16_ring_across_ok(int64_t K, int64_t ld) {
  return ld >= 1 && ld % 8 == 0 && K * ld * 2 < kPastEnd;
}

adahop_status bf16_ring_launch(const uint16_t* a, int a_across, int64_t lda, const uint16_t* b,
                               int b_across, int64_t ldb, int64_t m, int64_t n, int64_t K, void* C,
                               int64_t ldc, int out_f32, void* scratch, size_t scratch_bytes,
                               hipStream_t stream, hipEvent_t main_done) {
  if (!bf16_ring_ok(m, n, K) || ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15u))
    return fail(ADAHOP_ERR_UNSUPPORTED, "bf16 ring: K % 128 != 0, too long or misaligned operands");
  if ((a_across && (lda < m || !bf16_ring_across_ok(K, lda))) ||
      (b_across && (ldb < n || !bf16_ring_across_ok(K, ldb))))
    return fail(ADAHOP_ERR_UNSUPPORTED, "bf16 ring: an operand stored across K needs ld % 8 == 0, "
                                        "ld >= its rows of C and under 2 GiB");
  const adahop_status st = check_scratch(scratch, scratch_bytes, bf16_ring_scratch_bytes(m, n, K));
  if (st != ADAHOP_OK) return st;
  GemmArgs g{};
  g.a_codes = reinterpret_cast<const uint8_t*>(a);
  g.b_codes = reinterpret_cast<const uint8_t*>(b);
  g.a_ldb = 2 * lda;
  g.b_ldb = 2 * ldb;
  g.m = m; g.n = n; g.K = K; g.C = C; g.ldc = ldc; g.out_f32 = out_f32;
  g.tiles_m = (int)((m + BM - 1) / BM); g.tiles_n = (int)((n + BN - 1) / BN);
  g.oe_mode = 0;
  g.vec_ok = (ldc % (out_f32 ? 4 : 8) == 0) && ((reinterpret_cast<uintptr_t>(C) & 15u) == 0);
  const TailSplit ts = tail_split(m, n, K / 32);
  g.split_full = (int)ts.full;
  g.split_count = (int)ts.split;
  g.split_parts = ts.parts;
  g.split_ws = ts.split ? static_cast<float*>(scratch) : nullptr;
  const int64_t items = ts.full + ts.split * ts.parts, cus = device_cus();
  const dim3 rgrid((unsigned)(items < cus ? items : cus));
  if (a_across && b_across)
    gemm_mx_ring8_kernel<false, true, true, true><<<rgrid, dim3(kRing8Threads), 0, stream>>>(g);
  else if (a_across)
    gemm_mx_ring8_kernel<false, true, true, false><<<rgrid, dim3(kRing8Threads), 0, stream>>>(g);
  else if (b_across)
    gemm_mx_ring8_kernel<false, true, false, true><<<rgrid, dim3(kRing8Threads), 0, stream>>>(g);
  else
    gemm_mx_ring8_kernel<false, true><<<rgrid, dim3(kRing8Threads), 0, stream>>>(g);
  {
    const adahop_status ls = record_main_done(main_done, stream, "bf16 ring");
    if (ls != ADAHOP_OK) return ls;
  }
  if (ts.split) {
    const adahop_status ls = check_launch("bf16 ring");
    if (ls != ADAHOP_OK) return ls;
    gemm_split_fixup_kernel<<<dim3((unsigned)(ts.split * (BM / kFixRows))), dim3(kFixThreads), 0,
                              stream>>>(g);
  }
  return check_launch("bf16 ring");
}

namespace {
// dst[c][r] = src[r][c] for a bf16 [rows, cols] matrix (leading dim ld);
// dst is [cols, rows], leading dim rows. 64 x 64 tiles through LDS: thread t
// copies 16-byte chunk t % 8 of tile rows t / 8 and t / 8 + 32 in, then
// writes the 8 tile rows 8 (t % 8) .. +7 of tile columns t / 8 and t / 8 +
// 32 out. Chunk q of tile row r sits at chunk q ^ ((r / 8) % 8), so the
// column reads of a wave (8 rows 8 apart, one chunk group each) fall in
// distinct banks.
constexpr int kTT = 64;
__global__ void __launch_bounds__(256)
bf16_transpose_kernel(const uint16_t* __restrict__ src, int64_t rows, int64_t cols, int64_t ld,
                      uint16_t* __restrict__ dst, int vec_in, int vec_out) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTT * kTT];
  const int64_t r0 = (int64_t)blockIdx.x * kTT, c0 = (int64_t)blockIdx.y * kTT;
  const int t = threadIdx.x, q = t & 7, rr = t >> 3;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = rr + 32 * h;
    const int64_t gr = r0 + r, gc = c0 + 8 * q;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (gr < rows) {
      if (vec_in && gc + 8 <= cols) {
        v = *reinterpret_cast<const uint4*>(src + gr * ld + gc);
      } else {
        uint16_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = gc + j < cols ? src[gr * ld + gc + j] : 0;
        v = make_uint4(e[0] | (uint32_t)e[1] << 16, e[2] | (uint32_t)e[3] << 16,
                       e[4] | (uint32_t)e[5] << 16, e[6] | (uint32_t)e[7] << 16);
      }
    }
    *reinterpret_cast<uint4*>(&tile[r * kTT + 8 * (q ^ ((r >> 3) & 7))]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = rr + 32 * h;
    const int64_t gc = c0 + c, gr = r0 + 8 * q;
    if (gc >= cols) continue;
    uint16_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = tile[(8 * q + j) * kTT + 8 * ((c >> 3) ^ q) + (c & 7)];
    uint16_t* out = dst + gc * rows + gr;
    if (vec_out && gr + 8 <= rows) {
      *reinterpret_cast<uint4*>(out) =
          make_uint4(e[0] | (uint32_t)e[1] << 16, e[2] | (uint32_t)e[3] << 16,
                     e[4] | (uint32_t)e[5] << 16, e[6] | (uint32_t)e[7] << 16);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (gr + j < rows) out[j] = e[j];
    }
  }
}
}  // namespace

bool bf16_transpose_fits(int64_t rows, int64_t cols) {
  return rows >= 1 && cols >= 1 && (rows + kTT - 1) / kTT <= 0x7FFFFFFF && (cols + kTT - 1) / kTT <= 65535;
}

adahop_status bf16_transpose_launch(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld,
                                    uint16_t* dst, hipStream_t stream) {
  if (ld < cols || !bf16_transpose_fits(rows, cols))
    return fail(ADAHOP_ERR_UNSUPPORTED, "bf16 transpose: bad or too large shape");
  const int64_t gx = (rows + kTT - 1) / kTT, gy = (cols + kTT - 1) / kTT;
  const int vec_in = ld % 8 == 0 && (reinterpret_cast<uintptr_t>(src) & 15u) == 0;
  const int vec_out = rows % 8 == 0 && (reinterpret_cast<uintptr_t>(dst) & 15u) == 0;
  bf16_transpose_kernel<<<dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream>>>(
      src, rows, cols, ld, dst, vec_in, vec_out);
  return check_launch("bf16 transpose");
}

}  // namespace adahop
