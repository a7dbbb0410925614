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
// Tiling: a workgroup of 4 waves computes a 256 x 128 tile of C; each wave a
//   128 x 64 sub-tile (4 x 2 MFMA blocks, 128 fp32 accumulators per lane).
//   K advances 128 elements (64 bytes per row) per stage; stages are double
//   buffered in LDS (A 16 KB + B 8 KB per stage), the next stage's global loads
//   are in flight while the current one feeds the matrix cores. 16-byte chunks
//   of a row are XOR-swizzled in LDS so a wave's 16-byte fragment reads hit
//   distinct banks. Workgroup ids are remapped so that each XCD (ids i, i+8,
//   ...) works on a contiguous band of tiles that share operand rows in its L2.
// Outlier product: bf16 matrix cores (v_mfma_f32_32x32x16_bf16), 64 x 64
//   tiles, K split across workgroups into fp32 partials; the FP4 kernel's
//   epilogue sums a line's partials in a fixed order and adds them to the
//   fp32 accumulators before the single rounding to the output type (the
//   scatter-add). Inner extraction (rank-k term on every output) runs as extra
//   bf16 MFMAs on the tile's own accumulators. No atomics: results are
//   deterministic.
#include <utility>

#include "adahop_internal.h"

namespace adahop {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
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
constexpr int BM = 256, BN = 128;
constexpr int BKB = 64;                 // bytes of packed codes per row per stage (128 elements)
constexpr int kGemmThreads = 256;
constexpr int WM = 128, WN = 64;        // wave sub-tile
constexpr int FM = WM / 32, FN = WN / 32;
constexpr int kLdsA = BM * BKB, kLdsB = BN * BKB;

// 16-byte chunk c (0..3) of LDS row r lives at chunk c ^ swz(r).
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

struct GemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  int64_t m, n, K;
  void* C;
  int64_t ldc;
  int out_f32;
  int tiles_m, tiles_n;
  // outlier epilogue
  int oe_mode;
  int oe_k;
  const int32_t* oe_idx;
  const float* oe_partials;
  int oe_splits;
  const uint16_t* ia_ptr; int64_t ia_ld; int ia_inner;   // OE_INNER a: (i, p)
  const uint16_t* ib_ptr; int64_t ib_ld; int ib_inner;   // OE_INNER b: (j, p)
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

// KAligned: K % 128 == 0, so every stage is whole and a row's 4 scale bytes of
// a stage form one aligned dword.
template <bool KAligned>
__global__ void __launch_bounds__(kGemmThreads, 2) gemm_mx_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][kLdsA];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2][kLdsB];
  __shared__ uint8_t s_sa[2][BM * 4];
  __shared__ uint8_t s_sb[2][BN * 4];
  __shared__ int s_pos[BM > BN ? BM : BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware tile order: hardware places workgroup i on XCD i % 8; give each
  // XCD a contiguous run of tiles (row-major over tiles_n), so that its L2 sees
  // the same A rows.
  const int ntiles = g.tiles_m * g.tiles_n;
  int pid = blockIdx.x;
  {
    const int per = (ntiles + 7) / 8;
    const int xcd = pid & 7, local = pid >> 3;
    const int remapped = xcd * per + local;
    // Fall back to the identity when the last XCD band is short.
    pid = (ntiles % 8 == 0) ? remapped : pid;
  }
  const int tm = pid / g.tiles_n, tn = pid % g.tiles_n;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t Kb = g.K / 2;          // bytes per packed row
  const int64_t Ks = g.K / 32;         // scale bytes per row
  const int nk = (int)((g.K + 127) / 128);

  // Global -> register staging: A 4 chunks, B 2 chunks of 16 bytes per thread.
  uint4 ra[4], rb[2];
  uint32_t rsa = 0, rsb = 0;
  // A stage's 4 scale bytes of one row; past K they read as 0 (their codes are 0 too).
  auto load_scales = [&](const uint8_t* sc, int64_t row, int64_t sb0) -> uint32_t {
    if (KAligned) return *reinterpret_cast<const uint32_t*>(sc + row * Ks + sb0);
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t col = sb0 + q < Ks ? sb0 + q : Ks - 1;
      const uint32_t b = sc[row * Ks + col];
      v |= (sb0 + q < Ks ? b : 0u) << (8 * q);
    }
    return v;
  };
  auto load_stage = [&](int kt) {
    const int64_t kb0 = (int64_t)kt * BKB;
    const int c = tid & 3;
    const bool kin = KAligned || kb0 + c * 16 < Kb;
    const int64_t kc = kin ? kb0 + c * 16 : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t row = m0 + (tid >> 2) + 64 * i;
      row = row < g.m ? row : g.m - 1;
      const uint4 q = *reinterpret_cast<const uint4*>(g.a_codes + row * Kb + kc);
      ra[i] = kin ? q : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int64_t row = n0 + (tid >> 2) + 64 * i;
      row = row < g.n ? row : g.n - 1;
      const uint4 q = *reinterpret_cast<const uint4*>(g.b_codes + row * Kb + kc);
      rb[i] = kin ? q : make_uint4(0, 0, 0, 0);
    }
    const int64_t sb0 = (int64_t)kt * 4;
    {
      int64_t row = m0 + tid;
      rsa = load_scales(g.a_scales, row < g.m ? row : g.m - 1, sb0);
    }
    {
      int64_t row = n0 + (tid & (BN - 1));
      rsb = load_scales(g.b_scales, row < g.n ? row : g.n - 1, sb0);
    }
  };
  auto store_stage = [&](int buf) {
    const int c = tid & 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 2) + 64 * i;
      *reinterpret_cast<uint4*>(&s_a[buf][r * BKB + ((c ^ swz(r)) << 4)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (tid >> 2) + 64 * i;
      *reinterpret_cast<uint4*>(&s_b[buf][r * BKB + ((c ^ swz(r)) << 4)]) = rb[i];
    }
    *reinterpret_cast<uint32_t*>(&s_sa[buf][tid * 4]) = rsa;
    if (tid < BN) *reinterpret_cast<uint32_t*>(&s_sb[buf][tid * 4]) = rsb;
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  load_stage(0);
  store_stage(0);
  __syncthreads();

  const int lrow = lane & 31, khalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_stage(kt + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = ks * 2 + khalf;
      v8i fa[FM], fb[FN];
      int sa[FM], sb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WM + i * 32 + lrow;
        const uint4 q = *reinterpret_cast<const uint4*>(&s_a[buf][r * BKB + ((c ^ swz(r)) << 4)]);
        fa[i] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
        sa[i] = s_sa[buf][r * 4 + c];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * WN + j * 32 + lrow;
        const uint4 q = *reinterpret_cast<const uint4*>(&s_b[buf][r * BKB + ((c ^ swz(r)) << 4)]);
        fb[j] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
        sb[j] = s_sb[buf][r * 4 + c];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[i], fb[j], acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
    }
    // Keep the next stage's LDS stores (which wait for its global loads) after
    // this stage's matrix-core work, so the load latency overlaps the MFMAs.
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
  }

  // Inner extraction: C += a[:, 0:k] * b[:, 0:k]^T on bf16 matrix cores,
  // 16 extracted lines per MFMA (lane: row l%32, lines 8*(l/32) .. +7).
  if (g.oe_mode == ADAHOP_ROUTE_OE_INNER) {
    for (int p0 = 0; p0 < g.oe_k; p0 += 16) {
      v8bf fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        int64_t row = m0 + wm * WM + i * 32 + lrow;
        row = row < g.m ? row : g.m - 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int p = p0 + 8 * khalf + e;
          const uint16_t h = p < g.oe_k ? view_at(g.ia_ptr, g.ia_ld, g.ia_inner, row, p) : 0;
          fa[i][e] = __builtin_bit_cast(__bf16, h);
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        int64_t col = n0 + wn * WN + j * 32 + lrow;
        col = col < g.n ? col : g.n - 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int p = p0 + 8 * khalf + e;
          const uint16_t h = p < g.oe_k ? view_at(g.ib_ptr, g.ib_ld, g.ib_inner, col, p) : 0;
          fb[j][e] = __builtin_bit_cast(__bf16, h);
        }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }

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
      for (int q = tid; q < span; q += kGemmThreads) s_pos[q] = -1;
      __syncthreads();
      for (int p = lo + tid; p < hi; p += kGemmThreads) s_pos[g.oe_idx[p] - lo_v] = p;
      __syncthreads();
    }
  }

  const int64_t pstride = oe_rows ? (int64_t)g.oe_k * g.n : g.m * (int64_t)g.oe_k;
  static_for<FM>([&](auto I) {
    static_for<FN>([&](auto J) {
      const int lc = wn * WN + J * 32 + lrow;
      const int64_t col = n0 + lc;
      static_for<16>([&](auto V) {
        const int lr = wm * WM + I * 32 + acc_row(V, lane);
        const int64_t row = m0 + lr;
        float val = acc[I][J][(int)V];
        if (any_oe) {
          const int p = s_pos[oe_rows ? lr : lc];
          if (p >= 0 && row < g.m && col < g.n) {
            const int64_t off = oe_rows ? (int64_t)p * g.n + col : row * g.oe_k + p;
            float sum = 0.0f;
            for (int sp = 0; sp < g.oe_splits; ++sp) sum += g.oe_partials[sp * pstride + off];
            val += sum;
          }
        }
        if (row < g.m && col < g.n) {
          if (g.out_f32)
            static_cast<float*>(g.C)[row * g.ldc + col] = val;
          else
            static_cast<uint16_t*>(g.C)[row * g.ldc + col] = f32_to_bf16_rne(val);
        }
      });
    });
  });
}

// ---------------------------------------------------------------------------
// bf16 product on matrix cores: P[x][y] = sum_t X(x,t) * Y(y,t), split over K.
// 64 x 64 tile, 4 waves of 32 x 32, K stage 64, LDS rows padded to 72
// elements. Loads follow the memory order of each view (contiguous along t
// for inner-contiguous views, along x otherwise) so that a wave's loads are
// coalesced either way.
// ---------------------------------------------------------------------------
constexpr int OT = 64, OK = 64, OPAD = 72, kOeThreads = 256;

struct OeArgs {
  const uint16_t* x; int64_t xld; int xin;
  const uint16_t* y; int64_t yld; int yin;
  int64_t nx, ny, K, kchunk;
  float* partials;                 // [splits][nx][ny], or nullptr
  void* C; int64_t ldc; int out_f32;   // direct output when partials == nullptr
};

__device__ __forceinline__ void load_tile_bf16(uint16_t* s, const uint16_t* p, int64_t ld,
                                               int inner, int64_t r0, int64_t nr, int64_t t0,
                                               int64_t t1) {
  const int tid = threadIdx.x;
  for (int e = tid; e < OT * OK; e += kOeThreads) {
    int r, t;
    if (inner) { r = e / OK; t = e % OK; } else { t = e / OT; r = e % OT; }
    const int64_t gr = r0 + r, gt = t0 + t;
    uint16_t h = 0;
    if (gr < nr && gt < t1) h = inner ? p[gr * ld + gt] : p[gt * ld + gr];
    s[r * OPAD + t] = h;
  }
}

__global__ void __launch_bounds__(kOeThreads) oe_product_kernel(OeArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t sx[OT * OPAD];
  __shared__ __attribute__((aligned(16))) uint16_t sy[OT * OPAD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wx = wave >> 1, wy = wave & 1;
  const int64_t x0 = (int64_t)blockIdx.x * OT, y0 = (int64_t)blockIdx.y * OT;
  const int64_t tb = (int64_t)blockIdx.z * g.kchunk;
  const int64_t te = (tb + g.kchunk < g.K) ? tb + g.kchunk : g.K;
  v16f acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  for (int64_t t0 = tb; t0 < te; t0 += OK) {
    __syncthreads();
    load_tile_bf16(sx, g.x, g.xld, g.xin, x0, g.nx, t0, te);
    load_tile_bf16(sy, g.y, g.yld, g.yin, y0, g.ny, t0, te);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < OK; ks += 16) {
      const int off = ks + 8 * (lane >> 5);
      const uint4 qa = *reinterpret_cast<const uint4*>(&sx[(wx * 32 + (lane & 31)) * OPAD + off]);
      const uint4 qb = *reinterpret_cast<const uint4*>(&sy[(wy * 32 + (lane & 31)) * OPAD + off]);
      const v8bf fa = __builtin_bit_cast(v8bf, qa);
      const v8bf fb = __builtin_bit_cast(v8bf, qb);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc, 0, 0, 0);
    }
  }
  const int64_t col = y0 + wy * 32 + (lane & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t row = x0 + wx * 32 + acc_row(v, lane);
    if (row >= g.nx || col >= g.ny) continue;
    if (g.partials) {
      g.partials[(int64_t)blockIdx.z * g.nx * g.ny + row * g.ny + col] = acc[v];
    } else if (g.out_f32) {
      static_cast<float*>(g.C)[row * g.ldc + col] = acc[v];
    } else {
      static_cast<uint16_t*>(g.C)[row * g.ldc + col] = f32_to_bf16_rne(acc[v]);
    }
  }
}

}  // namespace

int oe_splits(int64_t nx, int64_t ny, int64_t K) {
  const int64_t tiles = ((nx + OT - 1) / OT) * ((ny + OT - 1) / OT);
  int64_t s = (512 + tiles - 1) / tiles;
  const int64_t smax = K / 256 > 0 ? K / 256 : 1;   // at least 256 K per split
  if (s > smax) s = smax;
  if (s > 64) s = 64;
  return (int)(s < 1 ? 1 : s);
}

static int64_t kchunk_for(int64_t K, int splits) {
  int64_t c = (K + splits - 1) / splits;
  return (c + OK - 1) / OK * OK;
}

adahop_status oe_product_launch(Bf16View X, Bf16View Y, int64_t nx, int64_t ny, int64_t K,
                                int splits, float* partials, hipStream_t stream) {
  OeArgs a{X.ptr, X.ld, X.inner_contiguous, Y.ptr, Y.ld, Y.inner_contiguous, nx, ny, K,
           kchunk_for(K, splits), partials, nullptr, 0, 0};
  const dim3 grid((unsigned)((nx + OT - 1) / OT), (unsigned)((ny + OT - 1) / OT), (unsigned)splits);
  oe_product_kernel<<<grid, dim3(kOeThreads), 0, stream>>>(a);
  return check_launch("oe_product");
}

adahop_status bf16_gemm_launch(Bf16View X, Bf16View Y, int64_t m, int64_t n, int64_t K,
                               void* C, int64_t ldc, int out_f32, hipStream_t stream) {
  const int64_t gx = (m + OT - 1) / OT, gy = (n + OT - 1) / OT;
  if (gx > 0x7FFFFFFF || gy > 65535) return fail(ADAHOP_ERR_UNSUPPORTED, "bf16 gemm: too large");
  OeArgs a{X.ptr, X.ld, X.inner_contiguous, Y.ptr, Y.ld, Y.inner_contiguous, m, n, K, K,
           nullptr, C, ldc, out_f32};
  oe_product_kernel<<<dim3((unsigned)gx, (unsigned)gy, 1), dim3(kOeThreads), 0, stream>>>(a);
  return check_launch("bf16_gemm");
}

adahop_status gemm_mx_launch(const uint8_t* a_codes, const uint8_t* a_scales,
                             const uint8_t* b_codes, const uint8_t* b_scales, int64_t m,
                             int64_t n, int64_t K, const OeEpilogue& oe, void* C, int64_t ldc,
                             int out_f32, hipStream_t stream) {
  const int64_t tiles_m = (m + BM - 1) / BM, tiles_n = (n + BN - 1) / BN;
  if (tiles_m * tiles_n > 0x7FFFFFFF) return fail(ADAHOP_ERR_UNSUPPORTED, "gemm: too large");
  GemmArgs g{};
  g.a_codes = a_codes; g.a_scales = a_scales; g.b_codes = b_codes; g.b_scales = b_scales;
  g.m = m; g.n = n; g.K = K; g.C = C; g.ldc = ldc; g.out_f32 = out_f32;
  g.tiles_m = (int)tiles_m; g.tiles_n = (int)tiles_n;
  g.oe_mode = oe.mode; g.oe_k = oe.k; g.oe_idx = oe.idx; g.oe_partials = oe.partials;
  g.oe_splits = oe.splits;
  g.ia_ptr = oe.a.ptr; g.ia_ld = oe.a.ld; g.ia_inner = oe.a.inner_contiguous;
  g.ib_ptr = oe.b.ptr; g.ib_ld = oe.b.ld; g.ib_inner = oe.b.inner_contiguous;
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(kGemmThreads);
  const bool scales4 = ((reinterpret_cast<uintptr_t>(a_scales) | reinterpret_cast<uintptr_t>(b_scales)) & 3u) == 0;
  if (K % 128 == 0 && scales4)
    gemm_mx_kernel<true><<<grid, block, 0, stream>>>(g);
  else
    gemm_mx_kernel<false><<<grid, block, 0, stream>>>(g);
  return check_launch("gemm_mx");
}

}  // namespace adahop
