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
// Selection without a host round trip and without atomics, by radix select
// on the fp64 score bits (scores are >= 0, so their bit patterns order like
// the values): a workgroup holds 4 or 16 scores per thread in registers, and
// 16 passes of 4-bit digits (per-thread packed counters, wave and workgroup
// sums) narrow down the k-th largest score; once the digit bin holding it has
// at most 256 scores, those are ranked exactly one against all. Every score above T
// is kept, and of the scores equal to T the ones with the lowest indices --
// the key (score descending, index ascending) is a strict total order, so
// the result is unique. A prefix sum over the threads, which own the
// candidates in index order, writes the kept indices already sorted. Levels
// of many workgroups first cut every chunk of 1024 candidates (4096 when
// k > 256) to its best k, until one workgroup can take the rest.
#include <climits>

#include "adahop_internal.h"

#pragma clang fp contract(off)

namespace adahop {
namespace {

constexpr int kVarThreads = 256;
constexpr int kProbe = 64;


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

constexpr int kSelThreads = 256;
constexpr int kExact = 256;   // a digit bin this small is ranked exactly

// Exclusive prefix sum of v over the workgroup's threads in order; *total
// receives the sum. Uses s_tmp[THREADS / 64].
template <int THREADS>
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  int before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < THREADS / 64; ++w) {
    const int t = s_tmp[w];
    before += w < wave ? t : 0;
    sum += t;
  }
  __syncthreads();
  *total = sum;
  return before + x - v;
}

// One selection over entries (in_var[i], in_idx ? in_idx[i] : i), i < count,
// in chunks of THREADS * KPT per workgroup (KPT entries per thread); entries
// with a negative score are padding. Non-final: the chunk's best k entries (all of them if it has
// fewer, then padding) go to out_var/out_idx + blockIdx.x * k in index order.
// Final (one workgroup): the best k indices go to final_idx in ascending
// order (k <= the number of real entries, checked on the host).
template <int THREADS, int KPT>
__global__ void __launch_bounds__(THREADS)
foid_select_kernel(const double* __restrict__ in_var, const int32_t* __restrict__ in_idx,
                   int64_t count, int k, double* __restrict__ out_var,
                   int32_t* __restrict__ out_idx, int32_t* __restrict__ final_idx) {
  constexpr int kWaves = THREADS / 64;
  __shared__ uint32_t s_cnt[kWaves][16];
  __shared__ uint32_t s_tot[16];
  __shared__ uint64_t s_ekey[kExact];
  __shared__ int s_epos[kExact];
  __shared__ uint8_t s_esel[kExact];
  __shared__ int s_tmp[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t first = (int64_t)blockIdx.x * THREADS * KPT + (int64_t)tid * KPT;

  uint64_t key[KPT];
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int64_t g = first + j;
    const double v = g < count ? in_var[g] : -1.0;
    key[j] = (uint64_t)__double_as_longlong(v);
    valid |= (v >= 0.0 ? 1u : 0u) << j;
  }
  int nvalid;
  block_exclusive_scan<THREADS>(__popc(valid), s_tmp, &nvalid);

  // T = the k-th largest key; krem = how many keys equal to T are kept.
  uint64_t prefix = 0, pmask = 0;
  int krem = k;
  bool exact = false;   // the k-th key's bin, once small, is ranked exactly
  if (nvalid > k) {
    for (int pass = 0; pass < 16; ++pass) {
      const int shift = 60 - 4 * pass;
        uint64_t c[4] = {0, 0, 0, 0};   // 16 counters of 16 bits: digit d in c[d / 4]
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const bool in = ((valid >> j) & 1u) && (key[j] & pmask) == prefix;
        const int d = (int)((key[j] >> shift) & 15u);
        const uint64_t inc = in ? (1ull << (16 * (d & 3))) : 0ull;
        c[0] += (d >> 2) == 0 ? inc : 0ull;
        c[1] += (d >> 2) == 1 ? inc : 0ull;
        c[2] += (d >> 2) == 2 ? inc : 0ull;
        c[3] += (d >> 2) == 3 ? inc : 0ull;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
        for (int q = 0; q < 4; ++q) c[q] += __shfl_xor(c[q], off);
      }
      if (lane == 0) {
#pragma unroll
        for (int d = 0; d < 16; ++d) s_cnt[wave][d] = (uint32_t)((c[d >> 2] >> (16 * (d & 3))) & 0xFFFFu);
      }
      __syncthreads();
      if (tid < 16) {
        uint32_t t = 0;
        for (int w = 0; w < kWaves; ++w) t += s_cnt[w][tid];
        s_tot[tid] = t;
      }
      __syncthreads();
      // The digit of the k-th largest key among those matching the prefix.
      int cum = 0, dsel = 0;
      bool found = false;
#pragma unroll
      for (int d = 15; d >= 0; --d) {
        const int t = (int)s_tot[d];
        if (!found) {
          if (cum + t >= krem) { dsel = d; found = true; } else { cum += t; }
        }
      }
      krem -= cum;
      prefix |= (uint64_t)dsel << shift;
      pmask |= 15ull << shift;
      const int m = (int)s_tot[dsel];     // keys in the chosen bin
      __syncthreads();
      if (m <= kExact) { exact = true; break; }   // the same for every thread
    }
  } else {
    krem = 0;          // keep every real entry
  }

  uint32_t keep = 0;
  if (exact) {
    // Keys in a higher bin are kept; of the m keys in the bin, the krem best
    // by (key descending, position ascending), ranked one against all.
    uint32_t in = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (!((valid >> j) & 1u)) continue;
      const uint64_t b = key[j] & pmask;
      if (b > prefix) keep |= 1u << j;
      else if (b == prefix) in |= 1u << j;
    }
    int m;
    int p = block_exclusive_scan<THREADS>(__popc(in), s_tmp, &m);
    const int p0 = p;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (!((in >> j) & 1u)) continue;
      s_ekey[p] = key[j];
      s_epos[p] = tid * KPT + j;
      ++p;
    }
    __syncthreads();
    for (int t = tid; t < m; t += THREADS) {
      const uint64_t kt = s_ekey[t];
      const int pt = s_epos[t];
      int rank = 0;
      for (int u = 0; u < m; ++u) {
        const uint64_t ku = s_ekey[u];
        rank += (ku > kt || (ku == kt && s_epos[u] < pt)) ? 1 : 0;
      }
      s_esel[t] = rank < krem ? 1 : 0;
    }
    __syncthreads();
    p = p0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (!((in >> j) & 1u)) continue;
      if (s_esel[p]) keep |= 1u << j;
      ++p;
    }
  } else {
    // Kept: real keys above T, and the first krem keys equal to T in index order.
    uint32_t eq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (!((valid >> j) & 1u)) continue;
      if (nvalid <= k || key[j] > prefix) keep |= 1u << j;
      else if (key[j] == prefix) eq |= 1u << j;
    }
    int eq_total;
    const int eq_before = block_exclusive_scan<THREADS>(__popc(eq), s_tmp, &eq_total);
    int take = krem - eq_before;
    take = take < 0 ? 0 : take;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (((eq >> j) & 1u) && take > 0) { keep |= 1u << j; --take; }
    }
  }
  int kept;
  int pos = block_exclusive_scan<THREADS>(__popc(keep), s_tmp, &kept);

  if (final_idx != nullptr) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (!((keep >> j) & 1u)) continue;
      const int64_t g = first + j;
      final_idx[pos++] = in_idx ? in_idx[g] : (int32_t)g;
    }
    return;
  }
  const int64_t ob = (int64_t)blockIdx.x * k;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (!((keep >> j) & 1u)) continue;
    const int64_t g = first + j;
    out_var[ob + pos] = __longlong_as_double((long long)key[j]);
    out_idx[ob + pos] = in_idx ? in_idx[g] : (int32_t)g;
    ++pos;
  }
  for (int p = kept + tid; p < k; p += THREADS) {      // fewer than k real entries
    out_var[ob + p] = -1.0;
    out_idx[ob + p] = INT_MAX;
  }
}

// A level keeps k of every chunk of level_chunk(k) >= 4 k entries; the final
// workgroup takes up to 1024 entries (4 per thread), or 4096 when k > 256.
int64_t level_chunk(int32_t k) { return k <= 256 ? 1024 : 4096; }
int64_t final_cap(int32_t k) { return k <= 256 ? 1024 : 4096; }
int64_t chunks_of(int64_t n, int32_t k) { return (n + level_chunk(k) - 1) / level_chunk(k); }

adahop_status launch_select(bool final_level, const double* in_var, const int32_t* in_idx,
                            int64_t count, int32_t k, double* out_var, int32_t* out_idx,
                            int32_t* final_idx, hipStream_t stream) {
  const bool big = k > 256;
  const unsigned nb = final_level ? 1u : (unsigned)chunks_of(count, k);
  if (big)
    foid_select_kernel<kSelThreads, 16><<<nb, kSelThreads, 0, stream>>>(in_var, in_idx, count, k,
                                                                        out_var, out_idx, final_idx);
  else
    foid_select_kernel<kSelThreads, 4><<<nb, kSelThreads, 0, stream>>>(in_var, in_idx, count, k,
                                                                       out_var, out_idx, final_idx);
  return check_launch("foid_select");
}

}  // namespace

size_t foid_workspace_bytes(int64_t ncand, int32_t k) {
  const size_t var_bytes = align_up(sizeof(double) * (size_t)ncand, kAlign);
  if (ncand <= final_cap(k)) return var_bytes;
  const size_t entries = (size_t)chunks_of(ncand, k) * (size_t)k;
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
  if (ncand <= final_cap(k))
    return launch_select(true, var, nullptr, ncand, k, nullptr, nullptr, idx_out, stream);
  const size_t entries = (size_t)chunks_of(ncand, k) * (size_t)k;
  double* var_buf[2];
  int32_t* idx_buf[2];
  for (int b = 0; b < 2; ++b) {
    var_buf[b] = reinterpret_cast<double*>(p);
    p += align_up(entries * sizeof(double), kAlign);
    idx_buf[b] = reinterpret_cast<int32_t*>(p);
    p += align_up(entries * sizeof(int32_t), kAlign);
  }
  // Each level divides the count by at least 4, until one workgroup can take
  // the rest.
  const double* in_var = var;
  const int32_t* in_idx = nullptr;
  int64_t count = ncand;
  int cur = 0;
  while (count > final_cap(k)) {
    st = launch_select(false, in_var, in_idx, count, k, var_buf[cur], idx_buf[cur], nullptr, stream);
    if (st != ADAHOP_OK) return st;
    count = chunks_of(count, k) * k;
    in_var = var_buf[cur];
    in_idx = idx_buf[cur];
    cur ^= 1;
  }
  return launch_select(true, in_var, in_idx, count, k, nullptr, nullptr, idx_out, stream);
}

}  // namespace adahop
