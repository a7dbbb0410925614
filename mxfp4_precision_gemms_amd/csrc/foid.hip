// FOID (Fast Outlier Index Detection) for gfx950.
//
// "AdaHOP ..." (arXiv 2604.02525), appendix kernel 1 and Fig. 9: each
// candidate row or column is scored by the variance of its first 64 elements
// and the k highest-scoring lines become the outlier lines.
//
// Scores: one thread per candidate, fp64, two passes in index order (sum ->
// mean -> sum of squared deviations), each operation separately rounded, so
// the score is bit-identical to a sequential evaluation. Candidate columns
// are read coalesced (consecutive lanes = consecutive columns); a candidate
// row is one 128-byte run, read as 8 16-byte loads when aligned. With the
// full 64-element probe the values stay in registers between the two passes.
//
// Selection without a host round trip and without atomics: a workgroup sorts
// up to 2048 (score, index) pairs in LDS with a bitonic network on the key
// (score descending, index ascending) -- a strict total order, so the result
// is unique -- and keeps its best k. The survivors of all workgroups form the
// next level; when at most 2048 remain one workgroup takes the best k and
// sorts their indices ascending. Each level divides the count by 2048 / k.
#include <climits>

#include "adahop_internal.h"

#pragma clang fp contract(off)

namespace adahop {
namespace {

constexpr int kVarThreads = 256;
constexpr int kSelThreads = 256;
constexpr int kChunk = 2048;           // >= 2 * max k, so every level shrinks
constexpr int kProbe = 64;

__device__ __forceinline__ bool before(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__device__ __forceinline__ double bf16_to_f64(uint32_t h) {
  return (double)__uint_as_float(h << 16);
}

// Variance of candidate lines; var[l] for l < ncand.
__global__ void __launch_bounds__(kVarThreads)
foid_var_kernel(const uint16_t* __restrict__ t, int64_t ld, int axis, int P, int64_t ncand,
                double* __restrict__ var) {
  const int64_t l = (int64_t)blockIdx.x * kVarThreads + threadIdx.x;
  if (l >= ncand) return;
  if (P == kProbe) {
    // Values in registers: 32 dwords of bf16 pairs.
    uint32_t w[kProbe / 2];
    if (axis == ADAHOP_AXIS_ROWS && (ld & 7) == 0 && (reinterpret_cast<uintptr_t>(t) & 15) == 0) {
#pragma unroll
      for (int q = 0; q < kProbe / 8; ++q) {
        const uint4 v = *reinterpret_cast<const uint4*>(t + l * ld + 8 * q);
        w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kProbe; i += 2) {
        const uint32_t a = axis == ADAHOP_AXIS_ROWS ? t[l * ld + i] : t[(int64_t)i * ld + l];
        const uint32_t b = axis == ADAHOP_AXIS_ROWS ? t[l * ld + i + 1] : t[(int64_t)(i + 1) * ld + l];
        w[i / 2] = a | (b << 16);
      }
    }
    double sum = 0.0;
#pragma unroll
    for (int i = 0; i < kProbe; ++i) sum += bf16_to_f64((w[i / 2] >> (16 * (i & 1))) & 0xFFFFu);
    const double mean = sum / (double)kProbe;
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < kProbe; ++i) {
      const double d = bf16_to_f64((w[i / 2] >> (16 * (i & 1))) & 0xFFFFu) - mean;
      ss += d * d;
    }
    var[l] = ss / (double)kProbe;
    return;
  }
  double sum = 0.0;
  for (int i = 0; i < P; ++i)
    sum += bf16_to_f64(axis == ADAHOP_AXIS_ROWS ? t[l * ld + i] : t[(int64_t)i * ld + l]);
  const double mean = sum / (double)P;
  double ss = 0.0;
  for (int i = 0; i < P; ++i) {
    const double d =
        bf16_to_f64(axis == ADAHOP_AXIS_ROWS ? t[l * ld + i] : t[(int64_t)i * ld + l]) - mean;
    ss += d * d;
  }
  var[l] = ss / (double)P;
}

// Sorts s_var/s_idx[0..n) (n a power of two) so that the best entry comes first.
__device__ void bitonic_sort_desc(double* s_var, int* s_idx, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int e = threadIdx.x; e < n / 2; e += kSelThreads) {
        const int i = 2 * stride * (e / stride) + (e % stride);
        const int j = i + stride;
        const bool best_first = (i & size) == 0;
        const double vi = s_var[i], vj = s_var[j];
        const int ii = s_idx[i], ij = s_idx[j];
        const bool swap = best_first ? before(vj, ij, vi, ii) : before(vi, ii, vj, ij);
        if (swap) {
          s_var[i] = vj; s_var[j] = vi;
          s_idx[i] = ij; s_idx[j] = ii;
        }
      }
    }
  }
  __syncthreads();
}

// Ascending sort of s_key[0..n), n a power of two.
__device__ void bitonic_sort_int_asc(int* s_key, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int e = threadIdx.x; e < n / 2; e += kSelThreads) {
        const int i = 2 * stride * (e / stride) + (e % stride);
        const int j = i + stride;
        const bool up = (i & size) == 0;
        const int a = s_key[i], b = s_key[j];
        if (up ? (a > b) : (a < b)) { s_key[i] = b; s_key[j] = a; }
      }
    }
  }
  __syncthreads();
}

__device__ __forceinline__ int pow2_at_least(int v) {
  int n = 1;
  while (n < v) n <<= 1;
  return n;
}

// One selection level over `count` entries: (in_var[i], in_idx ? in_idx[i] : i).
// Each workgroup keeps the best k of its chunk (sentinels where it has fewer)
// at out + blockIdx.x * k, or, with final_idx set (one workgroup), writes the
// best k indices in ascending order.
__global__ void __launch_bounds__(kSelThreads)
foid_select_kernel(const double* __restrict__ in_var, const int32_t* __restrict__ in_idx,
                   int64_t count, int k, double* __restrict__ out_var,
                   int32_t* __restrict__ out_idx, int32_t* __restrict__ final_idx) {
  __shared__ double s_var[kChunk];
  __shared__ int s_idx[kChunk];
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  const int valid = (int)(count - base < kChunk ? count - base : kChunk);
  const int n = pow2_at_least(valid > k ? valid : k);
  for (int slot = threadIdx.x; slot < n; slot += kSelThreads) {
    const int64_t g = base + slot;
    if (slot < valid) {
      s_var[slot] = in_var[g];
      s_idx[slot] = in_idx ? in_idx[g] : (int)g;
    } else {
      s_var[slot] = -1.0;       // scores are >= 0, so sentinels sort last
      s_idx[slot] = INT_MAX;
    }
  }
  bitonic_sort_desc(s_var, s_idx, n);

  if (final_idx == nullptr) {
    for (int p = threadIdx.x; p < k; p += kSelThreads) {
      out_var[(int64_t)blockIdx.x * k + p] = s_var[p];
      out_idx[(int64_t)blockIdx.x * k + p] = s_idx[p];
    }
    return;
  }
  // Final: the first k entries are real candidates (k <= candidates, checked
  // on the host). Sort their indices ascending in place (the same thread reads
  // and writes each slot, so s_idx can hold the keys).
  const int kp = pow2_at_least(k);
  for (int p = threadIdx.x; p < kp; p += kSelThreads)
    if (p >= k) s_idx[p] = INT_MAX;
  bitonic_sort_int_asc(s_idx, kp);
  for (int p = threadIdx.x; p < k; p += kSelThreads) final_idx[p] = s_idx[p];
}

int64_t chunks_of(int64_t n) { return (n + kChunk - 1) / kChunk; }

}  // namespace

size_t foid_workspace_bytes(int64_t ncand, int32_t k) {
  const size_t var_bytes = align_up(sizeof(double) * (size_t)ncand, kAlign);
  if (ncand <= kChunk) return var_bytes;
  const size_t entries = (size_t)chunks_of(ncand) * (size_t)k;
  return var_bytes +
         2 * (align_up(entries * sizeof(double), kAlign) + align_up(entries * sizeof(int32_t), kAlign));
}

adahop_status foid_launch(const uint16_t* t, int64_t rows, int64_t cols, int64_t ld, int axis,
                          int32_t probe, int32_t k, int32_t* idx_out, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  const int64_t ncand = axis == ADAHOP_AXIS_ROWS ? rows : cols;
  const int64_t len = axis == ADAHOP_AXIS_ROWS ? cols : rows;
  const int P = (int)(probe < len ? probe : len);
  const size_t need = foid_workspace_bytes(ncand, k);
  if (ws == nullptr || ws_bytes < need)
    return fail(ADAHOP_ERR_WORKSPACE, "adahop_detect: workspace too small (need " +
                                          std::to_string(need) + " bytes)");
  char* p = static_cast<char*>(ws);
  double* var = reinterpret_cast<double*>(p);
  p += align_up(sizeof(double) * (size_t)ncand, kAlign);
  const int64_t vblocks = (ncand + kVarThreads - 1) / kVarThreads;
  if (vblocks > 0x7FFFFFFF) return fail(ADAHOP_ERR_UNSUPPORTED, "adahop_detect: too many candidates");
  foid_var_kernel<<<dim3((unsigned)vblocks), dim3(kVarThreads), 0, stream>>>(t, ld, axis, P, ncand,
                                                                              var);
  adahop_status st = check_launch("foid_var");
  if (st != ADAHOP_OK) return st;
  const dim3 block(kSelThreads);
  if (ncand <= kChunk) {
    foid_select_kernel<<<1, block, 0, stream>>>(var, nullptr, ncand, k, nullptr, nullptr, idx_out);
    return check_launch("foid_select");
  }
  const size_t entries = (size_t)chunks_of(ncand) * (size_t)k;
  double* var_buf[2];
  int32_t* idx_buf[2];
  for (int b = 0; b < 2; ++b) {
    var_buf[b] = reinterpret_cast<double*>(p);
    p += align_up(entries * sizeof(double), kAlign);
    idx_buf[b] = reinterpret_cast<int32_t*>(p);
    p += align_up(entries * sizeof(int32_t), kAlign);
  }
  // Level 0 reads the scores with implicit indices; later levels read survivors.
  int64_t nb = chunks_of(ncand);
  foid_select_kernel<<<dim3((unsigned)nb), block, 0, stream>>>(var, nullptr, ncand, k, var_buf[0],
                                                               idx_buf[0], nullptr);
  st = check_launch("foid_select");
  if (st != ADAHOP_OK) return st;
  int cur = 0;
  int64_t count = nb * k;
  while (count > kChunk) {
    nb = chunks_of(count);
    foid_select_kernel<<<dim3((unsigned)nb), block, 0, stream>>>(
        var_buf[cur], idx_buf[cur], count, k, var_buf[cur ^ 1], idx_buf[cur ^ 1], nullptr);
    st = check_launch("foid_select");
    if (st != ADAHOP_OK) return st;
    cur ^= 1;
    count = nb * k;
  }
  foid_select_kernel<<<1, block, 0, stream>>>(var_buf[cur], idx_buf[cur], count, k, nullptr,
                                              nullptr, idx_out);
  return check_launch("foid_select");
}

}  // namespace adahop
