// FOID (Fast Outlier Index Detection) for gfx950.
//
// "AdaHOP ..." (arXiv 2604.02525), appendix kernel 1 and Fig. 9: each
// candidate row or column is scored by the variance of its first 64 elements
// and the k highest-scoring lines become the outlier lines.
//
// Scores: one thread per candidate, fp64, two passes in index order (sum ->
// mean -> sum of squared deviations), each operation separately rounded, so
// that the score is bit-identical to a sequential evaluation. Candidate
// columns are read coalesced (consecutive lanes = consecutive columns);
// candidate rows are a 128-byte run each.
//
// Selection without a host round trip and without atomics: a workgroup sorts
// up to 4096 (score, index) pairs in LDS with a bitonic network on the key
// (score descending, index ascending) -- a strict total order, so the result
// is unique -- and keeps its best k. The survivors of all workgroups form the
// next level; when at most 4096 remain one workgroup takes the best k and
// sorts their indices ascending. Each level divides the count by 4096/k.
#include <climits>

#include "adahop_internal.h"

#pragma clang fp contract(off)

namespace adahop {
namespace {

constexpr int kThreads = 1024;
constexpr int kChunk = 4096;
constexpr int kPerThread = kChunk / kThreads;

__device__ __forceinline__ bool before(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__device__ __forceinline__ double bf16_to_f64(uint16_t h) {
  return (double)__uint_as_float((uint32_t)h << 16);
}

// Sorts s_var/s_idx[0..kChunk) so that the best entry comes first.
__device__ void bitonic_sort_desc(double* s_var, int* s_idx) {
  for (int size = 2; size <= kChunk; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int e = threadIdx.x; e < kChunk / 2; e += kThreads) {
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

// Ascending sort of s_key[0..n), n a power of two <= kChunk.
__device__ void bitonic_sort_int_asc(int* s_key, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int e = threadIdx.x; e < n / 2; e += kThreads) {
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

// One level. Source: the tensor (in_var == nullptr; candidate c of this
// workgroup is line blockIdx.x*kChunk + c) or a survivor list of n_in entries.
// Output: the best k of the chunk to out_var/out_idx + blockIdx.x*k (sentinels
// where the chunk has fewer), or, if final_idx is set (one workgroup), the best
// k indices in ascending order.
__global__ void __launch_bounds__(kThreads)
foid_level_kernel(const uint16_t* __restrict__ t, int64_t ld, int axis, int P, int64_t ncand,
                  const double* __restrict__ in_var, const int32_t* __restrict__ in_idx,
                  int64_t n_in, int k, double* __restrict__ out_var,
                  int32_t* __restrict__ out_idx, int32_t* __restrict__ final_idx) {
  __shared__ double s_var[kChunk];
  __shared__ int s_idx[kChunk];
  const int64_t base = (int64_t)blockIdx.x * kChunk;

  for (int q = 0; q < kPerThread; ++q) {
    const int slot = threadIdx.x + q * kThreads;
    const int64_t g = base + slot;
    double var = -1.0;
    int idx = INT_MAX;
    if (in_var == nullptr) {
      if (g < ncand) {
        double sum = 0.0;
        for (int i = 0; i < P; ++i)
          sum += bf16_to_f64(axis == ADAHOP_AXIS_ROWS ? t[g * ld + i] : t[(int64_t)i * ld + g]);
        const double mean = sum / (double)P;
        double ss = 0.0;
        for (int i = 0; i < P; ++i) {
          const double d =
              bf16_to_f64(axis == ADAHOP_AXIS_ROWS ? t[g * ld + i] : t[(int64_t)i * ld + g]) - mean;
          ss += d * d;
        }
        var = ss / (double)P;
        idx = (int)g;
      }
    } else if (g < n_in) {
      var = in_var[g];
      idx = in_idx[g];
    }
    s_var[slot] = var;
    s_idx[slot] = idx;
  }
  bitonic_sort_desc(s_var, s_idx);

  if (final_idx == nullptr) {
    for (int p = threadIdx.x; p < k; p += kThreads) {
      out_var[(int64_t)blockIdx.x * k + p] = s_var[p];
      out_idx[(int64_t)blockIdx.x * k + p] = s_idx[p];
    }
    return;
  }
  // Final: indices of the best k, ascending. The chunk's first k entries are
  // real candidates (k <= number of candidates, checked on the host).
  int kpad = 1;
  while (kpad < k) kpad <<= 1;
  __shared__ int s_key[kChunk];
  for (int p = threadIdx.x; p < kpad; p += kThreads) s_key[p] = p < k ? s_idx[p] : INT_MAX;
  bitonic_sort_int_asc(s_key, kpad);
  for (int p = threadIdx.x; p < k; p += kThreads) final_idx[p] = s_key[p];
}

int64_t blocks_for(int64_t n) { return (n + kChunk - 1) / kChunk; }

}  // namespace

size_t foid_workspace_bytes(int64_t ncand, int32_t k) {
  if (ncand <= kChunk) return 0;
  const size_t entries = (size_t)blocks_for(ncand) * (size_t)k;
  return 2 * (align_up(entries * sizeof(double), kAlign) + align_up(entries * sizeof(int32_t), kAlign));
}

adahop_status foid_launch(const uint16_t* t, int64_t rows, int64_t cols, int64_t ld, int axis,
                          int32_t probe, int32_t k, int32_t* idx_out, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  const int64_t ncand = axis == ADAHOP_AXIS_ROWS ? rows : cols;
  const int64_t len = axis == ADAHOP_AXIS_ROWS ? cols : rows;
  const int P = (int)(probe < len ? probe : len);
  const dim3 block(kThreads);
  if (ncand <= kChunk) {
    foid_level_kernel<<<1, block, 0, stream>>>(t, ld, axis, P, ncand, nullptr, nullptr, 0, k,
                                               nullptr, nullptr, idx_out);
    return check_launch("foid");
  }
  const size_t need = foid_workspace_bytes(ncand, k);
  if (ws == nullptr || ws_bytes < need)
    return fail(ADAHOP_ERR_WORKSPACE, "adahop_detect: workspace too small (need " +
                                          std::to_string(need) + " bytes)");
  const size_t entries = (size_t)blocks_for(ncand) * (size_t)k;
  char* p = static_cast<char*>(ws);
  double* var_buf[2];
  int32_t* idx_buf[2];
  for (int b = 0; b < 2; ++b) {
    var_buf[b] = reinterpret_cast<double*>(p);
    p += align_up(entries * sizeof(double), kAlign);
    idx_buf[b] = reinterpret_cast<int32_t*>(p);
    p += align_up(entries * sizeof(int32_t), kAlign);
  }
  int64_t nb = blocks_for(ncand);
  foid_level_kernel<<<dim3((unsigned)nb), block, 0, stream>>>(
      t, ld, axis, P, ncand, nullptr, nullptr, 0, k, var_buf[0], idx_buf[0], nullptr);
  adahop_status st = check_launch("foid");
  if (st != ADAHOP_OK) return st;
  int cur = 0;
  int64_t count = nb * k;
  while (count > kChunk) {
    nb = blocks_for(count);
    foid_level_kernel<<<dim3((unsigned)nb), block, 0, stream>>>(
        nullptr, 0, axis, P, 0, var_buf[cur], idx_buf[cur], count, k, var_buf[cur ^ 1],
        idx_buf[cur ^ 1], nullptr);
    st = check_launch("foid");
    if (st != ADAHOP_OK) return st;
    cur ^= 1;
    count = nb * k;
  }
  foid_level_kernel<<<1, block, 0, stream>>>(nullptr, 0, axis, P, 0, var_buf[cur],
                                             idx_buf[cur], count, k, nullptr, nullptr, idx_out);
  return check_launch("foid");
}

}  // namespace adahop
