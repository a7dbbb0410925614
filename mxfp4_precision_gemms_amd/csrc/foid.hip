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
// The first selection level computes the scores itself, in registers. The
// score arithmetic (about 500 vector instructions per candidate) bounds
// that step, so with few candidates the level takes chunks of 256 or 512 on
// more workgroups, one candidate per thread, as long as their survivors
// still fit one final workgroup;
// line_scores_kernel writes every candidate's score out on its own (the
// pattern calibration's input).
//
// Selection without a host round trip, by radix select on the fp64 score
// bits (select_block and select_level in foid_select.h): 512-thread
// workgroups in foid_select_kernel, digit counts by wave ballots summed in
// LDS, one barrier per 4-bit digit. Every score
// above the k-th largest, T, is kept, and of the scores equal to T the ones
// with the lowest indices -- the key (score descending, index ascending) is
// a strict total order, so the result is unique. A prefix sum over the
// threads, which own the candidates in index order, writes the kept indices
// already sorted. Levels of many workgroups first cut every chunk of 1024
// candidates (the first level 256 or 512 when that leaves few enough
// survivors; 4096 when k > 256) to its best k, until one workgroup can take
// the rest.
//
// In a product whose other operand is quantized down its columns, the
// selection can share its launch with that quantization
// (foid_beside_quant_kernel, 256-thread workgroups, when it takes at most two
// levels and k <= 256): the selection's few workgroups run while the
// quantizer's workgroups stream that operand. The selection code is in foid_select.h,
// the quantizer's tiles in quant_tiles.h.
#include <type_traits>

#include "foid_select.h"
#include "quant_tiles.h"

#pragma clang fp contract(off)

namespace adahop {
namespace {

constexpr int kSelThreads = 512;

template <int KPT, int FKPT = KPT>
__global__ void __launch_bounds__(kSelThreads) foid_select_kernel(SelectArgs a, SelectArgs fin,
                                                                  unsigned* counter) {
  select_level<kSelThreads, KPT, FKPT>(a, fin, counter, blockIdx.x, gridDim.x);
}

__global__ void foid_zero_kernel(unsigned* counter) { *counter = 0u; }

// FOID's selection and the quantization of the operand it does not scan in
// one launch: workgroups 0 .. nsel - 1 run the selection (its first level,
// whose last workgroup to finish runs the final one; or a lone final level),
// the others the quantizer's tiles: column-direction (Rows false: gx tiles
// of columns per 32-row band) or row-direction (Rows: gx tiles of 4 rows x
// 1024 columns, as iht_quant_rowwise_kernel numbers them). The quantizer
// reads no index (its operand has no extracted lines), so the two parts
// share nothing but the launch: the selection, latency-bound on a few
// workgroups, runs while the quantizer streams its operand instead of before
// it. The selection's workgroups come first, so they are dispatched first.
static_assert(kColThreads == kRowThreads, "both quantizers' tiles take 256-thread workgroups");
template <int KPT, bool NT, bool Rows>
__global__ void __launch_bounds__(kColThreads)
foid_beside_quant_kernel(SelectArgs a, SelectArgs fin, unsigned* counter, unsigned nsel,
                         QuantBeside q, unsigned gx) {
  if (blockIdx.x < nsel) {
    select_level<kColThreads, KPT, 4>(a, fin, counter, blockIdx.x, nsel);
    return;
  }
  const unsigned b = blockIdx.x - nsel;
  const int kchunk = q.layout == ADAHOP_LAYOUT_KCHUNK ? 1 : 0;
  if constexpr (Rows)
    rowwise_tile(q.src, q.outer, q.K, q.ld, (int)((q.K + kRowChunk - 1) / kRowChunk), 1, nullptr, 0, 0,
                 q.codes, q.scales, nullptr, kchunk, NT ? 1 : 0, b);
  else
    colwise_tile<true, true, NT>(q.src, q.K, q.outer, q.ld, nullptr, 0, 0, q.codes, q.scales, nullptr,
                                 kchunk, b % gx, b / gx);
}

// Every candidate's score on its own: one thread per line, the same
// candidate_variance the selection levels fall back to.
__global__ void __launch_bounds__(256) line_scores_kernel(const uint16_t* __restrict__ t, int64_t ld,
                                                          int axis, int P, int64_t ncand,
                                                          double* __restrict__ out) {
  const int64_t l = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (l < ncand) out[l] = candidate_variance(t, ld, axis, P, l);
}

// A level keeps k of every chunk of level_chunk(k) >= 4 k entries; the final
// workgroup takes up to 1024 entries (2 per thread), or 4096 when k > 256.
int64_t level_chunk(int32_t k) { return k <= 256 ? 1024 : 4096; }
int64_t final_cap(int32_t k) { return k <= 256 ? 1024 : 4096; }
// The first level's chunk: 256 or 512 candidates (one per thread) when
// that many chunks still leave at most final_cap survivors, else
// level_chunk.
int64_t first_chunk(int64_t n, int32_t k) {
  if (k <= 256) {
    for (int64_t c = 256; c <= 512; c *= 2)
      if (c >= 4 * (int64_t)k && (n + c - 1) / c * k <= final_cap(k)) return c;
  }
  return level_chunk(k);
}
int64_t chunks_of(int64_t n, int64_t chunk) { return (n + chunk - 1) / chunk; }

adahop_status launch_select(bool final_level, const SelectArgs& a, const SelectArgs& fin,
                            unsigned* counter, hipStream_t stream) {
  const unsigned nb = final_level ? 1u : (unsigned)chunks_of(a.count, a.chunk);
  if (a.k > 256)
    foid_select_kernel<8><<<nb, kSelThreads, 0, stream>>>(a, fin, counter);
  else if (a.chunk <= kSelThreads)
    foid_select_kernel<1, 2><<<nb, kSelThreads, 0, stream>>>(a, fin, counter);
  else
    foid_select_kernel<2><<<nb, kSelThreads, 0, stream>>>(a, fin, counter);
  return check_launch("foid_select");
}

}  // namespace

adahop_status line_scores_launch(const uint16_t* t, int64_t rows, int64_t cols, int64_t ld, int axis,
                                 int32_t probe, double* out, hipStream_t stream) {
  const int64_t ncand = axis == ADAHOP_AXIS_ROWS ? rows : cols;
  const int64_t len = axis == ADAHOP_AXIS_ROWS ? cols : rows;
  const int P = (int)(probe < len ? probe : len);
  const int64_t blocks = (ncand + 255) / 256;
  if (blocks > 0x7FFFFFFF) return fail(ADAHOP_ERR_UNSUPPORTED, "adahop_line_scores: too many lines");
  line_scores_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(t, ld, axis, P, ncand, out);
  return check_launch("line_scores");
}

bool foid_fits(int64_t ncand, int32_t k) {
  return ncand >= 1 && k >= 1 && chunks_of(ncand, first_chunk(ncand, k)) <= 0x7FFFFFFF;
}

size_t foid_workspace_bytes(int64_t ncand, int32_t k) {
  if (ncand <= final_cap(k)) return 0;
  // The levels' survivors, double buffered (level 0 scores in registers),
  // then the counter of the level that runs the final selection.
  const size_t entries = (size_t)chunks_of(ncand, first_chunk(ncand, k)) * (size_t)k;
  return 2 * (align_up(entries * sizeof(double), kAlign) + align_up(entries * sizeof(int32_t), kAlign)) +
         kAlign;
}

namespace {

// Whether q suits the quantizer tiles of its direction (the conditions
// iht_quant_launch applies to them; the column-direction tiles on their
// vectorized loads; the row-direction ones need 16-byte aligned rows of a
// multiple of 8 elements) and nsel selection workgroups plus q's tiles
// (gx x gy) fit one grid.
bool beside_grid(const QuantBeside& q, int64_t nsel, int64_t* gx, int64_t* gy) {
  if (q.K < 32 || q.K % 32 != 0 || q.outer < 1) return false;
  if (q.layout == ADAHOP_LAYOUT_KCHUNK &&
      (q.K % 128 != 0 || (reinterpret_cast<uintptr_t>(q.scales) & 3u) != 0))
    return false;
  if (q.contract == ADAHOP_AXIS_COLS) {
    if (q.ld % 8 != 0 || (reinterpret_cast<uintptr_t>(q.src) & 15u) != 0 || q.ld < q.K) return false;
    *gx = (q.outer + kRowRows - 1) / kRowRows * ((q.K + kRowChunk - 1) / kRowChunk);
    *gy = 1;
  } else {
    const bool vec = q.ld % 4 == 0 && (reinterpret_cast<uintptr_t>(q.src) & 7u) == 0 &&
                     (int64_t)kColBlocks * 32 * q.ld * 2 < 0x7FFFFFFF;
    if (!vec) return false;
    *gx = (q.outer + kColOut - 1) / kColOut;
    *gy = (q.K / 32 + kColBlocks - 1) / kColBlocks;
  }
  return *gx <= 0x7FFFFFFFLL / *gy && nsel + *gx * *gy <= 0x7FFFFFFFLL;
}

// Workgroups of FOID's selection when it fits one launch of 256-thread
// workgroups (k <= 256: a lone final level of up to 1024 candidates, or a
// first level whose survivors the final workgroup takes), else 0.
int64_t beside_selection_blocks(int64_t ncand, int32_t k) {
  if (k < 1 || k > 256 || ncand < 1) return 0;
  if (ncand <= final_cap(k)) return 1;
  const int64_t n = chunks_of(ncand, first_chunk(ncand, k));
  return n * k <= final_cap(k) ? n : 0;
}

// Launches FOID's selection (nsel workgroups: a lone final level, or the
// first level with the final one behind `counter`) together with q's
// quantization; the caller has checked beside_selection_blocks and
// beside_grid.
adahop_status launch_beside(const SelectArgs& a, const SelectArgs& fin, unsigned* counter,
                            int64_t nsel, const QuantBeside& q, hipStream_t stream) {
  int64_t gx = 0, gy = 0;
  if (!beside_grid(q, nsel, &gx, &gy) || a.chunk > 4 * kColThreads ||
      (counter && fin.chunk > 4 * kColThreads))
    return fail(ADAHOP_ERR_UNSUPPORTED, "foid: the quantization does not fit the selection's launch");
  if (counter) {
    foid_zero_kernel<<<1, 1, 0, stream>>>(counter);
    const adahop_status st = check_launch("foid_zero");
    if (st != ADAHOP_OK) return st;
  }
  const dim3 grid((unsigned)(nsel + gx * gy)), block(kColThreads);
  const unsigned ns = (unsigned)nsel, ugx = (unsigned)gx;
  auto go = [&](auto kpt, auto nt) {
    if (q.contract == ADAHOP_AXIS_COLS)
      foid_beside_quant_kernel<decltype(kpt)::value, decltype(nt)::value, true>
          <<<grid, block, 0, stream>>>(a, fin, counter, ns, q, ugx);
    else
      foid_beside_quant_kernel<decltype(kpt)::value, decltype(nt)::value, false>
          <<<grid, block, 0, stream>>>(a, fin, counter, ns, q, ugx);
  };
  using T1 = std::integral_constant<int, 1>;
  using T2 = std::integral_constant<int, 2>;
  using T4 = std::integral_constant<int, 4>;
  if (a.chunk <= kColThreads) {
    if (q.stream_src) go(T1{}, std::true_type{}); else go(T1{}, std::false_type{});
  } else if (a.chunk <= 2 * kColThreads) {
    if (q.stream_src) go(T2{}, std::true_type{}); else go(T2{}, std::false_type{});
  } else {
    if (q.stream_src) go(T4{}, std::true_type{}); else go(T4{}, std::false_type{});
  }
  return check_launch("foid_beside_quant");
}

}  // namespace

bool foid_beside_fits(int64_t ncand, int32_t k, const QuantBeside& q) {
  int64_t gx = 0, gy = 0;
  const int64_t nsel = beside_selection_blocks(ncand, k);
  return nsel > 0 && beside_grid(q, nsel, &gx, &gy);
}

adahop_status foid_launch(const uint16_t* t, int64_t rows, int64_t cols, int64_t ld, int axis,
                          int32_t probe, int32_t k, int32_t* idx_out, void* ws, size_t ws_bytes,
                          hipStream_t stream, const QuantBeside* beside, bool* beside_done) {
  if (beside_done) *beside_done = false;
  const int64_t ncand = axis == ADAHOP_AXIS_ROWS ? rows : cols;
  const int64_t len = axis == ADAHOP_AXIS_ROWS ? cols : rows;
  const int P = (int)(probe < len ? probe : len);
  const size_t need = foid_workspace_bytes(ncand, k);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(ADAHOP_ERR_WORKSPACE, "adahop_detect: workspace too small (need " +
                                          std::to_string(need) + " bytes)");
  if (!foid_fits(ncand, k))
    return fail(ADAHOP_ERR_UNSUPPORTED, "adahop_detect: too many candidates");
  SelectArgs a{t, ld, axis, P, nullptr, nullptr, ncand, k, nullptr, nullptr, nullptr, first_chunk(ncand, k)};
  const SelectArgs none{};
  const bool beside_ok = beside != nullptr && beside_done != nullptr &&
                         foid_beside_fits(ncand, k, *beside);
  if (ncand <= final_cap(k)) {
    a.chunk = final_cap(k);
    a.final_idx = idx_out;
    if (beside_ok) {
      *beside_done = true;
      return launch_beside(a, none, nullptr, 1, *beside, stream);
    }
    return launch_select(true, a, none, nullptr, stream);
  }
  const size_t entries = (size_t)chunks_of(ncand, a.chunk) * (size_t)k;
  char* p = static_cast<char*>(ws);
  double* var_buf[2];
  int32_t* idx_buf[2];
  for (int b = 0; b < 2; ++b) {
    var_buf[b] = reinterpret_cast<double*>(p);
    p += align_up(entries * sizeof(double), kAlign);
    idx_buf[b] = reinterpret_cast<int32_t*>(p);
    p += align_up(entries * sizeof(int32_t), kAlign);
  }
  unsigned* counter = reinterpret_cast<unsigned*>(p);
  // Each level divides the count by at least 4, until one workgroup can take
  // the rest; level 0 scores the candidates itself, and the last level before
  // the final one runs it too.
  int cur = 0;
  bool first = true;
  while (true) {
    a.out_var = var_buf[cur];
    a.out_idx = idx_buf[cur];
    const SelectArgs next{nullptr, 0, 0, 0, var_buf[cur], idx_buf[cur], chunks_of(a.count, a.chunk) * k, k,
                          nullptr, nullptr, nullptr, level_chunk(k)};
    if (next.count <= final_cap(k)) {
      SelectArgs fin = next;
      fin.final_idx = idx_out;
      if (first && beside_ok) {
        *beside_done = true;
        return launch_beside(a, fin, counter, chunks_of(a.count, a.chunk), *beside, stream);
      }
      foid_zero_kernel<<<1, 1, 0, stream>>>(counter);
      const adahop_status st = check_launch("foid_zero");
      if (st != ADAHOP_OK) return st;
      return launch_select(false, a, fin, counter, stream);
    }
    const adahop_status st = launch_select(false, a, none, nullptr, stream);
    if (st != ADAHOP_OK) return st;
    a = next;
    cur ^= 1;
    first = false;
  }
}

}  // namespace adahop
