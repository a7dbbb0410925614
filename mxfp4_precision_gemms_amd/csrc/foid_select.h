// FOID's scores and selection as device code (appendix kernel 1 and Fig. 9 of
// "AdaHOP ..." (arXiv 2604.02525)), included by foid.hip (the selection
// kernels) and iht_quant.hip (the selection beside the other operand's
// quantization in one launch). Workgroups of THREADS threads.
#pragma once

#include <climits>

#include "adahop_internal.h"

#pragma clang fp contract(off)

namespace adahop {
namespace {

constexpr int kProbe = 64;

__device__ __forceinline__ double bf16_to_f64(uint32_t h) {
  return (double)__uint_as_float(h << 16);
}

// Variance of candidate line l over its first P elements: fp64, two passes
// in index order (sum -> mean -> sum of squared deviations), each operation
// separately rounded.
// Out of line: the selection kernel calls it only off its fast path.
__device__ __attribute__((noinline)) double candidate_variance(const uint16_t* __restrict__ t, int64_t ld, int axis, int P,
                                     int64_t l) {
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
    // The packed words count as changed here, so the second pass converts
    // them again instead of keeping 64 fp64 values live.
#pragma unroll
    for (int i = 0; i < kProbe / 2; ++i) asm volatile("" : "+v"(w[i]));
    const double mean = sum / (double)kProbe;
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < kProbe; ++i) {
      const double d = bf16_to_f64((w[i / 2] >> (16 * (i & 1))) & 0xFFFFu) - mean;
      ss += d * d;
    }
    return ss / (double)kProbe;
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
  return ss / (double)P;
}

// Scores of the two adjacent candidates c, c + 1 with the full 64-element
// probe. Columns: each row is one 4-byte load holding both, so a wave reads
// 256 contiguous bytes per row; rows: 8 16-byte loads per row. Same
// operations, in the same order, as candidate_variance.
// `fence` marks the packed words as changed between the two passes, so the
// 128 fp64 conversions are redone rather than kept live in registers.
template <typename Lo, typename Hi, typename Fence>
__device__ __forceinline__ void pair_stats(Lo lo, Hi hi, Fence fence, double* v0, double* v1) {
  double s0 = 0.0, s1 = 0.0;
#pragma unroll
  for (int i = 0; i < kProbe; ++i) {
    s0 += bf16_to_f64(lo(i));
    s1 += bf16_to_f64(hi(i));
  }
  fence();
  const double m0 = s0 / (double)kProbe, m1 = s1 / (double)kProbe;
  double q0 = 0.0, q1 = 0.0;
#pragma unroll
  for (int i = 0; i < kProbe; ++i) {
    const double d0 = bf16_to_f64(lo(i)) - m0;
    const double d1 = bf16_to_f64(hi(i)) - m1;
    q0 += d0 * d0;
    q1 += d1 * d1;
  }
  *v0 = q0 / (double)kProbe;
  *v1 = q1 / (double)kProbe;
}

__device__ __forceinline__ void pair_variance(const uint16_t* __restrict__ t, int64_t ld, int axis,
                                              int64_t c, double* v0, double* v1) {
  if (axis == ADAHOP_AXIS_COLS) {
    uint32_t w[kProbe];
    const uint32_t* p = reinterpret_cast<const uint32_t*>(t + c);
#pragma unroll
    for (int i = 0; i < kProbe; ++i) w[i] = p[(int64_t)i * (ld / 2)];
    pair_stats([&](int i) { return w[i] & 0xFFFFu; }, [&](int i) { return w[i] >> 16; },
               [&]() {
#pragma unroll
                 for (int i = 0; i < kProbe; ++i) asm volatile("" : "+v"(w[i]));
               },
               v0, v1);
  } else {
    uint32_t r0[kProbe / 2], r1[kProbe / 2];
#pragma unroll
    for (int q = 0; q < kProbe / 8; ++q) {
      const uint4 a = *reinterpret_cast<const uint4*>(t + c * ld + 8 * q);
      const uint4 b = *reinterpret_cast<const uint4*>(t + (c + 1) * ld + 8 * q);
      r0[4 * q] = a.x; r0[4 * q + 1] = a.y; r0[4 * q + 2] = a.z; r0[4 * q + 3] = a.w;
      r1[4 * q] = b.x; r1[4 * q + 1] = b.y; r1[4 * q + 2] = b.z; r1[4 * q + 3] = b.w;
    }
    pair_stats([&](int i) { return (r0[i / 2] >> (16 * (i & 1))) & 0xFFFFu; },
               [&](int i) { return (r1[i / 2] >> (16 * (i & 1))) & 0xFFFFu; },
               [&]() {
#pragma unroll
                 for (int i = 0; i < kProbe / 2; ++i) asm volatile("" : "+v"(r0[i]), "+v"(r1[i]));
               },
               v0, v1);
  }
}

// Exclusive prefix sum of v, 0 <= v < 2^BITS, over the workgroup's threads
// in order; *total receives the sum. Within a wave by one ballot per bit of
// v and a count of the ballot's bits below the lane (no cross-lane shuffles,
// which go through the LDS); then over the waves. Uses s_tmp[THREADS / 64].
template <int THREADS, int BITS>
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = 0, wsum = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(((v >> b) & 1) != 0);
    x += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
    wsum += __popcll(m) << b;
  }
  if (lane == 0) s_tmp[wave] = wsum;
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
  return before + x;
}

// Inputs of one selection. Level 0 (t != nullptr) scores candidate lines
// [0, count) itself; later levels read (in_var[i], in_idx[i]), i < count,
// where a negative score is padding.
struct SelectArgs {
  const uint16_t* t; int64_t ld; int axis; int P;
  const double* in_var; const int32_t* in_idx;
  int64_t count;
  int k;
  double* out_var; int32_t* out_idx;   // non-final: k entries per workgroup
  int32_t* final_idx;                  // final (one workgroup): the k indices, ascending
  int64_t chunk;                       // entries per workgroup, <= THREADS x KPT
};

// Selection over chunks of a.chunk <= THREADS * KPT entries per workgroup,
// thread t owning entries a.chunk * b + KPT t .. + KPT - 1 in index order
// (threads past the chunk own none). Radix select
// on the fp64 score bits (scores are >= 0, so their bit patterns order like
// the values), 4 bits per pass from the top: each wave counts its keys in the
// current bin per next digit with ballots and writes the 16 counts to LDS,
// one barrier publishes the 8 x 16 counts, and every wave sums them and picks
// the digit of the krem-th largest key itself (integer counts: the order of
// the adds does not matter). The pass
// loop ends once the chosen bin holds exactly the keys still needed (all of
// them kept), else after 16 passes with T, the k-th largest key: every key
// above T is kept and, of the keys equal to T, the ones with the lowest
// indices -- the key (score descending, index ascending) is a strict total
// order, so the result is unique. A prefix sum over the threads writes the
// kept entries already sorted by index.
// Stores of survivors another workgroup reads in the same launch:
// agent-scope monotonic atomic stores, which write through this XCD's L2
// (on gfx950 an ordinary store may stay dirty in it, out of another XCD's
// sight).
__device__ __forceinline__ void publish(double* p, double v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int THREADS, int KPT>
__device__ __forceinline__ void select_block(const SelectArgs& a, int block,
                                             uint32_t (*s_cnt)[THREADS / 64][16], int* s_tmp,
                                             bool write_through = false) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t first = (int64_t)block * a.chunk + (int64_t)tid * KPT;
  const int64_t cend = (int64_t)block * a.chunk + a.chunk;
  const int64_t end = cend < a.count ? cend : a.count;

  double v[KPT];
  const bool pair = KPT == 2 && a.t && a.P == kProbe && first + 1 < end &&
                    (a.axis == ADAHOP_AXIS_COLS
                         ? (a.ld & 1) == 0 && (reinterpret_cast<uintptr_t>(a.t) & 3) == 0
                         : (a.ld & 7) == 0 && (reinterpret_cast<uintptr_t>(a.t) & 15) == 0);
  if (pair) {
    pair_variance(a.t, a.ld, a.axis, first, &v[0], &v[KPT - 1]);
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int64_t g = first + j;
      v[j] = -1.0;
      if (g < end) v[j] = a.t ? candidate_variance(a.t, a.ld, a.axis, a.P, g) : a.in_var[g];
    }
  }
  uint64_t key[KPT];
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    key[j] = (uint64_t)__double_as_longlong(v[j]);
    valid |= (v[j] >= 0.0 ? 1u : 0u) << j;
  }

  uint64_t prefix = 0, pmask = 0;
  int krem = a.k;
  bool keep_all = false, bin_kept = false;
  for (int pass = 0; pass < 16; ++pass) {
    const int shift = 60 - 4 * pass;
    const int buf = pass & 1;
    // The wave's count of each next digit among its keys in the current bin,
    // by ballots rather than LDS atomics (in the first passes every key of a
    // wave shares one digit, and adds to one counter serialize): per key
    // slot, a ballot of the keys in the bin and one of each digit bit; lane
    // d < 16 keeps the keys whose 4 bits spell d and counts them. Its row of
    // the pass's buffer is written once; the buffers alternate, so a row is
    // rewritten only after the barrier that ends every wave's reads of it.
    // (The ballot of a digit bit is taken on its own and masked with the
    // bin's ballot in scalar registers: a ballot of the conjunction compiles
    // to a select and a second compare per bit.)
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool in = ((valid >> j) & 1u) && (key[j] & pmask) == prefix;
      const uint32_t dj = (uint32_t)(key[j] >> shift) & 15u;
      const uint64_t inm = __builtin_amdgcn_ballot_w64(in);
      uint64_t m = inm;
#pragma unroll
      for (int bit = 0; bit < 4; ++bit) {
        const uint64_t bm = __builtin_amdgcn_ballot_w64((dj & (1u << bit)) != 0u) & inm;
        m &= ((lane >> bit) & 1) ? bm : ~bm;
      }
      mine += (uint32_t)__popcll(m);
    }
    if (lane < 16) s_cnt[buf][wave][lane] = mine;
    __syncthreads();
    int tot = 0;
    if (lane < 16) {
#pragma unroll
      for (int w = 0; w < THREADS / 64; ++w) tot += (int)s_cnt[buf][w][lane];
    }
    // Lane d < 16: keys of the bin with next digit >= d (a suffix sum over
    // lanes d .. 15, which form one DPP row: four adds of the value 1, 2, 4
    // and 8 lanes up, 0 past the row's end). The digit of the krem-th
    // largest key is the largest d whose suffix holds at least krem keys;
    // the keys above it are those of digits d + 1 .. 15. Wave-uniform
    // throughout.
    int suf = tot;
    suf += __builtin_amdgcn_update_dpp(0, suf, 0x101, 0xF, 0xF, true);   // row_shl:1
    suf += __builtin_amdgcn_update_dpp(0, suf, 0x102, 0xF, 0xF, true);   // row_shl:2
    suf += __builtin_amdgcn_update_dpp(0, suf, 0x104, 0xF, 0xF, true);   // row_shl:4
    suf += __builtin_amdgcn_update_dpp(0, suf, 0x108, 0xF, 0xF, true);   // row_shl:8
    const int all = __builtin_amdgcn_readfirstlane(suf);
    if (pass == 0 && all <= a.k) { keep_all = true; break; }   // every real entry is kept
    const uint64_t ge = __builtin_amdgcn_ballot_w64(lane < 16 && suf >= krem);
    const int dsel = ge ? 63 - __builtin_clzll(ge) : 0;   // ge is never empty here
    const int m = __builtin_amdgcn_readlane(tot, dsel);
    const int cum = dsel < 15 ? __builtin_amdgcn_readlane(suf, dsel + 1) : 0;
    krem -= cum;
    prefix |= (uint64_t)dsel << shift;
    pmask |= 15ull << shift;
    if (m == krem) { bin_kept = true; break; }
  }

  uint32_t keep = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (!((valid >> j) & 1u)) continue;
    const uint64_t b = key[j] & pmask;
    if (keep_all || b > prefix || (bin_kept && b == prefix)) keep |= 1u << j;
    else if (!bin_kept && key[j] == prefix) eq |= 1u << j;
  }
  if (!keep_all && !bin_kept) {
    // All 16 digits decided: prefix is T; the first krem keys equal to T.
    int eq_total;
    const int eq_before = block_exclusive_scan<THREADS, KPT == 1 ? 1 : KPT == 2 ? 2 : 4>(__popc(eq), s_tmp, &eq_total);
    int take = krem - eq_before;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (((eq >> j) & 1u) && take > 0) { keep |= 1u << j; --take; }
    }
  }
  int kept;
  int pos = block_exclusive_scan<THREADS, KPT == 1 ? 1 : KPT == 2 ? 2 : 4>(__popc(keep), s_tmp, &kept);

  if (a.final_idx != nullptr) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (!((keep >> j) & 1u)) continue;
      const int64_t g = first + j;
      a.final_idx[pos++] = a.in_idx ? a.in_idx[g] : (int32_t)g;
    }
    return;
  }
  const int64_t ob = (int64_t)block * a.k;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (!((keep >> j) & 1u)) continue;
    const int64_t g = first + j;
    const double v = __longlong_as_double((long long)key[j]);
    const int32_t i = a.in_idx ? a.in_idx[g] : (int32_t)g;
    if (write_through) {
      publish(&a.out_var[ob + pos], v);
      publish(&a.out_idx[ob + pos], i);
    } else {
      a.out_var[ob + pos] = v;
      a.out_idx[ob + pos] = i;
    }
    ++pos;
  }
  for (int p = kept + tid; p < a.k; p += THREADS) {      // fewer than k real entries
    if (write_through) {
      publish(&a.out_var[ob + p], -1.0);
      publish(&a.out_idx[ob + p], (int32_t)INT_MAX);
    } else {
      a.out_var[ob + p] = -1.0;
      a.out_idx[ob + p] = INT_MAX;
    }
  }
}

// One level of selection, workgroup b taking chunk b. With `counter` (zero
// at launch), the level is the last before the final one, and the level's
// last workgroup to finish runs the final selection `fin` over all
// survivors: every workgroup writes its survivors through to memory
// (agent-scope stores), waits for them to complete, and only then counts
// itself in; the one that counts last invalidates its L2 (an acquire fence,
// no write-back) before reading them. No full-cache fence: one that writes
// back the L2 costs 2-11 us per workgroup while a quantizer's output sits
// dirty in it. No workgroup waits for another, and the final selection
// starts as soon as the level ends, without a second dispatch.
// `block` is this workgroup's chunk and `blocks` the level's number of
// workgroups (of THREADS threads).
template <int THREADS, int KPT, int FKPT = KPT>
__device__ __forceinline__ void select_level(const SelectArgs& a, const SelectArgs& fin,
                                             unsigned* counter, int block, unsigned blocks) {
  __shared__ uint32_t s_cnt[2][THREADS / 64][16];
  __shared__ int s_tmp[THREADS / 64];
  __shared__ int s_last;
  select_block<THREADS, KPT>(a, block, s_cnt, s_tmp, counter != nullptr);
  if (counter == nullptr) return;
  // Every thread's write-through stores complete before the workgroup counts
  // itself in (the compiler barriers keep the stores on their side).
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     blocks - 1 ? 1 : 0;
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  select_block<THREADS, FKPT>(fin, 0, s_cnt, s_tmp);
}

}  // namespace
}  // namespace adahop
