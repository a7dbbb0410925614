// Host side of the AdaHOP library: argument checks, routing, workspace plans
// and the launch sequence of one product. Every check runs before the first
// launch; the library never allocates or synchronizes.
#include <algorithm>
#include <climits>
#include <cstring>
#include <limits>
#include <mutex>
#include <string>
#include <vector>

#include "adahop_internal.h"

namespace adahop {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

adahop_status fail(adahop_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

adahop_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(ADAHOP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return ADAHOP_OK;
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Storage-frame description of one product (the textbook frame is C = A B).
struct OpShape {
  int64_t m, n, K;
  int64_t lhs_rows, lhs_cols, rhs_rows, rhs_cols;
  int lhs_contract, rhs_contract;   // axis of the stored tensor the contraction runs along
  bool lhs_transposed, rhs_transposed;   // textbook operand = stored tensor transposed
};

bool op_shape(adahop_op op, int64_t T, int64_t Din, int64_t Dout, OpShape* s) {
  switch (op) {
    case ADAHOP_OP_FWD:     // Y = X W^T: A = X, B = W^T
      *s = {T, Dout, Din, T, Din, Dout, Din, ADAHOP_AXIS_COLS, ADAHOP_AXIS_COLS, false, true};
      return true;
    case ADAHOP_OP_DGRAD:   // dX = GY W: A = GY, B = W
      *s = {T, Din, Dout, T, Dout, Dout, Din, ADAHOP_AXIS_COLS, ADAHOP_AXIS_ROWS, false, false};
      return true;
    case ADAHOP_OP_WGRAD:   // dW = GY^T X: A = GY^T, B = X
      *s = {Dout, Din, T, T, Dout, T, Din, ADAHOP_AXIS_ROWS, ADAHOP_AXIS_ROWS, true, false};
      return true;
  }
  return false;
}

adahop_pattern transposed(adahop_pattern p) {
  return p == ADAHOP_PAT_ROW ? ADAHOP_PAT_COL : p == ADAHOP_PAT_COL ? ADAHOP_PAT_ROW : p;
}

bool valid_pattern(int p) { return p >= ADAHOP_PAT_NONE && p <= ADAHOP_PAT_COL; }

// View of a stored [rows, cols] tensor as (outer, t) with t along `contract`.
Bf16View stored_view(const uint16_t* p, int64_t cols, int contract) {
  return {p, cols, contract == ADAHOP_AXIS_COLS ? 1 : 0};
}

// Length of a line of the lhs or rhs along `axis` (a row has cols elements).
int64_t line_len(const OpShape& s, bool lhs, int axis) {
  const int64_t rows = lhs ? s.lhs_rows : s.rhs_rows, cols = lhs ? s.lhs_cols : s.rhs_cols;
  return axis == ADAHOP_AXIS_ROWS ? cols : rows;
}

// Gathered lines (adahop_iht_quant layout): line-major [k][len], len = the
// source's cols for extracted rows, its rows for extracted columns. As (line
// p, position x along the line):
Bf16View lines_by_line(const uint16_t* g, int64_t len) { return Bf16View{g, len, 1}; }
// ... and as (position x, line p):
Bf16View lines_by_position(const uint16_t* g, int64_t len) { return Bf16View{g, len, 0}; }

struct Plan {
  adahop_plan pub;
  OpShape shape;
  bool zero_lhs = false, zero_rhs = false;
  int lhs_zero_axis = ADAHOP_AXIS_ROWS, rhs_zero_axis = ADAHOP_AXIS_ROWS;
  int splits = 0;
  // The outlier product formed in the other operand's quantization (one
  // read of it): its number of partial-sum groups, 0 when not used.
  int fused_groups = 0;
  size_t off_foid = SIZE_MAX, off_partials = SIZE_MAX, off_gemm = SIZE_MAX;
  size_t foid_bytes = 0, gemm_bytes = 0;
  // BF16 route on the ring kernel: whether it reads A / B across K, the
  // leading dimension of what it reads, and the workspace offset of a
  // transposed copy the operand is read from (SIZE_MAX: read in place).
  bool bf16_ring = false;
  bool a_across = false, b_across = false;
  int64_t a_ld = 0, b_ld = 0;
  size_t off_lhs_t = SIZE_MAX, off_rhs_t = SIZE_MAX;
  // The rhs (X of a weight gradient) comes from a saved forward context:
  // its indices, packed residual and lines are at these offsets of the
  // context buffer, and the workspace holds none of them.
  bool rhs_in_ctx = false;
  size_t ctx_off_idx = SIZE_MAX, ctx_off_codes = SIZE_MAX, ctx_off_scales = SIZE_MAX,
         ctx_off_lines = SIZE_MAX, ctx_bytes = 0;
};

constexpr size_t kNone = SIZE_MAX;

// The outer outlier product's factors of a plan (OE_LEFT: X the gathered
// rows of A, Y the rhs as stored; OE_RIGHT: X the lhs as stored, Y the
// gathered columns of B), on the given tensors and gathered lines.
void oe_views(const Plan& P, const uint16_t* lhs, const uint16_t* rhs, const uint16_t* ll,
              const uint16_t* rl, Bf16View* X, Bf16View* Y) {
  const OpShape& s = P.shape;
  if (P.pub.route == ADAHOP_ROUTE_OE_LEFT) {
    *X = lines_by_line(ll, line_len(s, true, P.lhs_zero_axis));       // (p, t)
    *Y = stored_view(rhs, s.rhs_cols, s.rhs_contract);               // (j, t)
  } else {
    *X = stored_view(lhs, s.lhs_cols, s.lhs_contract);               // (i, t)
    *Y = lines_by_line(rl, line_len(s, false, P.rhs_zero_axis));      // (p, t)
  }
}

adahop_status make_plan(adahop_op op, int64_t T, int64_t Din, int64_t Dout,
                        adahop_pattern pat_lhs, adahop_pattern pat_rhs, adahop_route_t route,
                        int32_t oe_rank, Plan* P, bool rhs_in_ctx = false,
                        bool oe_in_quant = false) {
  std::memset(&P->pub, 0, sizeof(P->pub));
  P->rhs_in_ctx = rhs_in_ctx;
  if (!op_shape(op, T, Din, Dout, &P->shape)) return fail(ADAHOP_ERR_INVALID, "invalid op");
  if (T < 1 || Din < 1 || Dout < 1) return fail(ADAHOP_ERR_INVALID, "sizes must be >= 1");
  if (!valid_pattern(pat_lhs) || !valid_pattern(pat_rhs))
    return fail(ADAHOP_ERR_INVALID, "invalid pattern");
  if (route == ADAHOP_ROUTE_AUTO) route = adahop_route(op, pat_lhs, pat_rhs);
  if (route < ADAHOP_ROUTE_BF16 || route > ADAHOP_ROUTE_MXFP4)
    return fail(ADAHOP_ERR_INVALID, "invalid route");
  const OpShape& s = P->shape;
  if (route != ADAHOP_ROUTE_BF16 && s.K % 32 != 0)
    return fail(ADAHOP_ERR_INVALID, "contraction length " + std::to_string(s.K) +
                                        " is not a multiple of 32");
  adahop_plan& pb = P->pub;
  if (rhs_in_ctx && (route == ADAHOP_ROUTE_BF16 || route == ADAHOP_ROUTE_OE_LEFT ||
                     route == ADAHOP_ROUTE_OE_INNER))
    return fail(ADAHOP_ERR_UNSUPPORTED, "a weight gradient on this route reads X in bf16: "
                                        "no context can stand in for it");
  pb.route = route;
  pb.m = s.m; pb.n = s.n; pb.K = s.K;
  pb.scan_tensor = -1;
  pb.scan_axis = ADAHOP_AXIS_ROWS;
  pb.layout = ADAHOP_LAYOUT_ROWS;
  pb.off_idx = pb.off_a_codes = pb.off_a_scales = pb.off_b_codes = pb.off_b_scales = kNone;
  pb.off_lhs_lines = pb.off_rhs_lines = kNone;
  if (route == ADAHOP_ROUTE_BF16) {
    // K % 128 == 0: the ring kernel on bf16 matrix cores. An operand not
    // contiguous along K ([K, cols] stored) is read in place when its row
    // length is a multiple of 8 and it is under 2 GiB, else transposed into
    // the workspace first.
    pb.ws_bytes = 0;
    if (bf16_ring_ok(s.m, s.n, s.K)) {
      size_t off = 0;
      auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes, kAlign); return o; };
      P->bf16_ring = true;
      P->a_ld = P->b_ld = s.K;
      if (s.lhs_contract == ADAHOP_AXIS_ROWS) {
        P->a_across = bf16_ring_across_ok(s.K, s.lhs_cols);
        P->a_ld = s.lhs_cols;
        if (!P->a_across) { P->off_lhs_t = take(2 * (size_t)s.m * (size_t)s.K); P->a_ld = s.K; }
      }
      if (s.rhs_contract == ADAHOP_AXIS_ROWS) {
        P->b_across = bf16_ring_across_ok(s.K, s.rhs_cols);
        P->b_ld = s.rhs_cols;
        if (!P->b_across) { P->off_rhs_t = take(2 * (size_t)s.n * (size_t)s.K); P->b_ld = s.K; }
      }
      // Both operands along K (the forward): the kernel reads an operand
      // across K faster (a load covers two 512-byte K-rows instead of 64
      // bytes of 16 rows: 2.81 against 3.14 ms for one 32768 x 14336 x 4096
      // product), so on large products the operand with fewer rows is
      // copied across K first; the copy reads and writes 4 bytes per
      // element, a few percent of the product's time when the other side
      // has 8192 rows or more.
      if (!P->a_across && !P->b_across && P->off_lhs_t == kNone && P->off_rhs_t == kNone &&
          std::max(s.m, s.n) >= 8192) {
        if (s.n <= s.m && bf16_ring_across_ok(s.K, s.n)) {
          P->off_rhs_t = take(2 * (size_t)s.n * (size_t)s.K);
          P->b_across = true;
          P->b_ld = s.n;
        } else if (s.m < s.n && bf16_ring_across_ok(s.K, s.m)) {
          P->off_lhs_t = take(2 * (size_t)s.m * (size_t)s.K);
          P->a_across = true;
          P->a_ld = s.m;
        }
      }
      P->gemm_bytes = bf16_ring_scratch_bytes(s.m, s.n, s.K);
      if (P->gemm_bytes) P->off_gemm = take(P->gemm_bytes);
      pb.ws_bytes = off;
      if ((P->off_lhs_t != kNone && !bf16_transpose_fits(s.lhs_rows, s.lhs_cols)) ||
          (P->off_rhs_t != kNone && !bf16_transpose_fits(s.rhs_rows, s.rhs_cols)))
        return fail(ADAHOP_ERR_UNSUPPORTED, "operand too wide for the K-major copy");
    }
    // The tile kernel that runs when the ring kernel does not apply.
    if (!oe_product_fits(s.m, s.n)) return fail(ADAHOP_ERR_UNSUPPORTED, "bf16 product too wide");
    return ADAHOP_OK;
  }

  const bool oe = route == ADAHOP_ROUTE_OE_LEFT || route == ADAHOP_ROUTE_OE_RIGHT ||
                  route == ADAHOP_ROUTE_OE_INNER;
  if (oe) {
    // OE_LEFT: rows of A; OE_RIGHT: columns of B; OE_INNER: A's columns (lhs
    // lines across its contraction axis) and the matching rows of B.
    if (route == ADAHOP_ROUTE_OE_LEFT) {
      pb.scan_tensor = 0;
      pb.scan_axis = (adahop_axis)(s.lhs_contract == ADAHOP_AXIS_COLS ? ADAHOP_AXIS_ROWS
                                                                       : ADAHOP_AXIS_COLS);
    } else if (route == ADAHOP_ROUTE_OE_RIGHT) {
      pb.scan_tensor = 1;
      pb.scan_axis = (adahop_axis)(s.rhs_contract == ADAHOP_AXIS_COLS ? ADAHOP_AXIS_ROWS
                                                                       : ADAHOP_AXIS_COLS);
    } else {
      pb.scan_tensor = 0;
      pb.scan_axis = (adahop_axis)s.lhs_contract;
    }
    const int64_t rows = pb.scan_tensor == 0 ? s.lhs_rows : s.rhs_rows;
    const int64_t cols = pb.scan_tensor == 0 ? s.lhs_cols : s.rhs_cols;
    const int64_t ncand = pb.scan_axis == ADAHOP_AXIS_ROWS ? rows : cols;
    if (oe_rank < 1 || oe_rank > ncand)
      return fail(ADAHOP_ERR_INVALID, "oe_rank " + std::to_string(oe_rank) +
                                          " outside [1, " + std::to_string(ncand) + "]");
    if (oe_rank > kMaxK) return fail(ADAHOP_ERR_UNSUPPORTED, "oe_rank above 1024");
    if (!foid_fits(ncand, oe_rank)) return fail(ADAHOP_ERR_UNSUPPORTED, "too many FOID candidates");
    pb.k = oe_rank;
    if (pb.scan_tensor == 0) { P->zero_lhs = true; P->lhs_zero_axis = pb.scan_axis; }
    else { P->zero_rhs = true; P->rhs_zero_axis = pb.scan_axis; }
    if (route == ADAHOP_ROUTE_OE_INNER) { P->zero_rhs = true; P->rhs_zero_axis = s.rhs_contract; }
    P->foid_bytes = foid_workspace_bytes(ncand, oe_rank);
  }

  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes, kAlign); return o; };
  if (rhs_in_ctx) {
    // Only a weight gradient whose route leaves X's lines alone or extracts
    // X's columns (FOID over X) can take X from a context: its indices,
    // packed residual and lines live there, laid out like this.
    if (op != ADAHOP_OP_WGRAD || P->zero_lhs)
      return fail(ADAHOP_ERR_UNSUPPORTED, "a context holds X for a weight gradient on route IHT, "
                                          "MXFP4 or OE_RIGHT only");
    size_t c = 0;
    auto ctake = [&](size_t bytes) { size_t o = c; c += align_up(bytes, kAlign); return o; };
    if (oe) P->ctx_off_idx = ctake(sizeof(int32_t) * (size_t)pb.k);
    P->ctx_off_codes = ctake((size_t)s.n * (size_t)(s.K / 2));
    P->ctx_off_scales = ctake((size_t)s.n * (size_t)(s.K / 32));
    if (P->zero_rhs)
      P->ctx_off_lines = ctake(2 * (size_t)pb.k * (size_t)line_len(s, false, P->rhs_zero_axis));
    P->ctx_bytes = c;
  } else if (oe) {
    pb.off_idx = take(sizeof(int32_t) * (size_t)pb.k);
    if (P->foid_bytes) P->off_foid = take(P->foid_bytes);
  }
  pb.off_a_codes = take((size_t)s.m * (size_t)(s.K / 2));
  pb.off_a_scales = take((size_t)s.m * (size_t)(s.K / 32));
  if (!rhs_in_ctx) {
    pb.off_b_codes = take((size_t)s.n * (size_t)(s.K / 2));
    pb.off_b_scales = take((size_t)s.n * (size_t)(s.K / 32));
  }
  if (P->zero_lhs) pb.off_lhs_lines = take(2 * (size_t)pb.k * (size_t)line_len(s, true, P->lhs_zero_axis));
  if (P->zero_rhs && !rhs_in_ctx)
    pb.off_rhs_lines = take(2 * (size_t)pb.k * (size_t)line_len(s, false, P->rhs_zero_axis));
  if (route == ADAHOP_ROUTE_OE_LEFT || route == ADAHOP_ROUTE_OE_RIGHT) {
    const int64_t nx = route == ADAHOP_ROUTE_OE_LEFT ? pb.k : s.m;
    const int64_t ny = route == ADAHOP_ROUTE_OE_LEFT ? s.n : pb.k;
    P->splits = oe_splits(nx, ny, s.K);
    // Room for the outlier product run either way: before the GEMM (its
    // partial sums and their sum) or inside it (partial sums and the
    // extracted lines' residuals), whichever the call's pointers allow.
    size_t bytes = sizeof(float) * (size_t)(P->splits + 1) * (size_t)nx * (size_t)ny;
    Bf16View X, Y;
    oe_views(*P, nullptr, nullptr, nullptr, nullptr, &X, &Y);
    const int fp = oe_fused_parts(s.m, s.n, s.K, route, pb.k, X, Y, false);
    if (fp > 0) bytes = std::max(bytes, oe_fused_bytes(s.m, s.n, route, pb.k, fp));
    // Asked for: the operand FOID does not scan, when it is quantized down
    // its columns, forms the outlier product in its quantization pass
    // (partial sums per group of K tiles, then their sum in order).
    const bool other_lhs = pb.scan_tensor == 1;
    if (oe_in_quant && !rhs_in_ctx &&
        (other_lhs ? s.lhs_contract : s.rhs_contract) == ADAHOP_AXIS_ROWS) {
      int tiles_per_wg = 0;
      P->fused_groups = iht_quant_oe_groups(s.K, other_lhs ? s.lhs_cols : s.rhs_cols, pb.k,
                                            &tiles_per_wg);
      if (P->fused_groups > 0)
        bytes = std::max(bytes, sizeof(float) * (size_t)(P->fused_groups + 1) * (size_t)nx * (size_t)ny);
    }
    pb.oe_in_quant = P->fused_groups > 0 ? 1 : 0;
    P->off_partials = take(bytes);
  }
  // Shapes a launcher would refuse are rejected here, before the call's
  // first launch.
  if (!iht_quant_fits(s.lhs_rows, s.lhs_cols, s.lhs_contract) ||
      !iht_quant_fits(s.rhs_rows, s.rhs_cols, s.rhs_contract) || !gemm_mx_fits(s.m, s.n))
    return fail(ADAHOP_ERR_UNSUPPORTED, "operands too large for the quantizer or GEMM grids");
  if (route == ADAHOP_ROUTE_OE_LEFT || route == ADAHOP_ROUTE_OE_RIGHT) {
    const int64_t nx = route == ADAHOP_ROUTE_OE_LEFT ? pb.k : s.m;
    const int64_t ny = route == ADAHOP_ROUTE_OE_LEFT ? s.n : pb.k;
    if (!oe_product_fits(nx, ny)) return fail(ADAHOP_ERR_UNSUPPORTED, "outlier product too wide");
  }
  // Operands the main GEMM kernel streams are packed K-chunked by the
  // quantizers; otherwise row-major, with the GEMM's own scale reordering.
  pb.layout = gemm_mx_kchunk_ok(s.m, s.n, s.K) ? ADAHOP_LAYOUT_KCHUNK : ADAHOP_LAYOUT_ROWS;
  P->gemm_bytes = gemm_mx_scratch_bytes(s.m, s.n, s.K, pb.layout);
  if (P->gemm_bytes) P->off_gemm = take(P->gemm_bytes);
  pb.ws_bytes = off;
  return ADAHOP_OK;
}

struct Events {
  void* const* ev;
  hipStream_t stream;
  hipEvent_t at(int i) const { return ev ? static_cast<hipEvent_t>(ev[i]) : nullptr; }
  adahop_status record(int i) const {
    if (!ev) return ADAHOP_OK;
    hipError_t e = hipEventRecord(static_cast<hipEvent_t>(ev[i]), stream);
    return e == hipSuccess ? ADAHOP_OK
                           : fail(ADAHOP_ERR_HIP, std::string("hipEventRecord: ") +
                                                      hipGetErrorString(e));
  }
};

#define ADAHOP_TRY(x)                      \
  do {                                     \
    adahop_status _st = (x);               \
    if (_st != ADAHOP_OK) return _st;      \
  } while (0)

// A second stream per device, for the quantization of the operand FOID does
// not scan, beside FOID and the stages after it.
// Created once per device at the default priority; `mu` is held from the
// fork to the join, so that concurrent calls on one device do not re-record
// the two events in between.
struct SideStream {
  std::mutex mu;
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool tried = false;
};
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];

// The current device's side stream, or nullptr if it cannot be had (the
// stages then run one after another on the caller's stream). Call with
// g_side[dev].mu held.
SideStream* side_stream_locked(int dev) {
  SideStream& ss = g_side[dev];
  if (!ss.tried) {
    ss.tried = true;
    if (hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      ss.stream = nullptr;
    }
  }
  return ss.stream ? &ss : nullptr;
}

adahop_status hip_ok(hipError_t e, const char* what) {
  return e == hipSuccess ? ADAHOP_OK : fail(ADAHOP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Held from the fork of the side stream to its join. However the call ends
// after the fork (an error included), the caller's stream waits for
// everything enqueued on the side stream before the device's lock is
// released: no work of the call outlives its return unordered, and a
// captured call never leaves the side stream forked.
struct SideJoin {
  SideStream* side = nullptr;
  hipStream_t stream = nullptr;
  std::unique_lock<std::mutex> lock;
  bool joined = false;
  adahop_status join() {
    if (!side || joined) return ADAHOP_OK;
    joined = true;
    adahop_status st = hip_ok(hipEventRecord(side->join, side->stream), "hipEventRecord");
    if (st == ADAHOP_OK) st = hip_ok(hipStreamWaitEvent(stream, side->join, 0), "hipStreamWaitEvent");
    return st;
  }
  ~SideJoin() {
    if (side && !joined) {
      // Error path: keep the message of the error being returned.
      const std::string msg = adahop_last_error();
      joined = true;
      if (hipEventRecord(side->join, side->stream) == hipSuccess)
        (void)hipStreamWaitEvent(stream, side->join, 0);
      (void)hipGetLastError();
      set_error(msg);
    }
  }
};

// A weight gradient's rhs taken from a saved forward context.
struct CtxIn {
  const uint8_t* base;
  size_t bytes;
};

adahop_status run_gemm(adahop_op op, const uint16_t* lhs, const uint16_t* rhs, int64_t T,
                       int64_t Din, int64_t Dout, adahop_pattern pat_lhs,
                       adahop_pattern pat_rhs, adahop_route_t route, int32_t oe_rank,
                       void* out, adahop_out_dtype out_dtype, void* ws, size_t ws_bytes,
                       hipStream_t stream, void* const* events, const CtxIn* ctx = nullptr,
                       bool oe_in_quant = false) {
  set_error("");
  if (!lhs || (!rhs && !ctx) || !out) return fail(ADAHOP_ERR_INVALID, "null lhs, rhs or out");
  if (out_dtype != ADAHOP_OUT_BF16 && out_dtype != ADAHOP_OUT_F32)
    return fail(ADAHOP_ERR_INVALID, "invalid out_dtype");
  Plan P;
  ADAHOP_TRY(make_plan(op, T, Din, Dout, pat_lhs, pat_rhs, route, oe_rank, &P, ctx != nullptr,
                       oe_in_quant));
  if (ctx) {
    if (!ctx->base) return fail(ADAHOP_ERR_INVALID, "null context");
    if (ctx->bytes < P.ctx_bytes)
      return fail(ADAHOP_ERR_INVALID, "context smaller than its plan: " + std::to_string(P.ctx_bytes) +
                                          " bytes");
    if (reinterpret_cast<uintptr_t>(ctx->base) & 15u)
      return fail(ADAHOP_ERR_UNSUPPORTED, "the context must be 16-byte aligned");
  }
  const adahop_plan& pb = P.pub;
  const OpShape& s = P.shape;
  if (pb.ws_bytes > 0 && (ws == nullptr || ws_bytes < pb.ws_bytes))
    return fail(ADAHOP_ERR_WORKSPACE, "workspace too small: need " + std::to_string(pb.ws_bytes) +
                                          " bytes");
  if (pb.route != ADAHOP_ROUTE_BF16) {
    const bool lhs_ok = s.lhs_contract == ADAHOP_AXIS_ROWS || (aligned16(lhs) && s.lhs_cols % 8 == 0);
    const bool rhs_ok = s.rhs_contract == ADAHOP_AXIS_ROWS || (aligned16(rhs) && s.rhs_cols % 8 == 0);
    if (!lhs_ok || !rhs_ok || (ws && !aligned16(ws)))
      return fail(ADAHOP_ERR_UNSUPPORTED,
                  "an operand quantized along its rows must be 16-byte aligned with a row length "
                  "% 8 == 0, and the workspace 16-byte aligned");
  }
  const Events E{events, stream};
  const int out_f32 = out_dtype == ADAHOP_OUT_F32 ? 1 : 0;
  ADAHOP_TRY(E.record(0));

  if (pb.route == ADAHOP_ROUTE_BF16) {
    ADAHOP_TRY(E.record(1));
    // The ring kernel needs 16-byte aligned operands and workspace; with
    // any of them misaligned the product runs on the tile kernel instead.
    const bool lhs_copy = P.off_lhs_t != kNone, rhs_copy = P.off_rhs_t != kNone;
    if (P.bf16_ring && (lhs_copy || aligned16(lhs)) && (rhs_copy || aligned16(rhs)) &&
        (pb.ws_bytes == 0 || aligned16(ws))) {
      char* w = static_cast<char*>(ws);
      const uint16_t* a = lhs;
      const uint16_t* b = rhs;
      if (lhs_copy) {
        uint16_t* t = reinterpret_cast<uint16_t*>(w + P.off_lhs_t);
        ADAHOP_TRY(bf16_transpose_launch(lhs, s.lhs_rows, s.lhs_cols, s.lhs_cols, t, stream));
        a = t;
      }
      ADAHOP_TRY(E.record(2));
      if (rhs_copy) {
        uint16_t* t = reinterpret_cast<uint16_t*>(w + P.off_rhs_t);
        ADAHOP_TRY(bf16_transpose_launch(rhs, s.rhs_rows, s.rhs_cols, s.rhs_cols, t, stream));
        b = t;
      }
      ADAHOP_TRY(E.record(3));
      ADAHOP_TRY(E.record(4));
      ADAHOP_TRY(bf16_ring_launch(a, P.a_across, P.a_ld, b, P.b_across, P.b_ld,
                                  s.m, s.n, s.K, out, s.n, out_f32,
                                  P.gemm_bytes ? w + P.off_gemm : nullptr, P.gemm_bytes, stream,
                                  E.at(5)));
      return E.record(6);
    }
    for (int i = 2; i <= 4; ++i) ADAHOP_TRY(E.record(i));
    ADAHOP_TRY(bf16_gemm_launch(stored_view(lhs, s.lhs_cols, s.lhs_contract),
                                stored_view(rhs, s.rhs_cols, s.rhs_contract), s.m, s.n, s.K, out,
                                s.n, out_f32, stream));
    ADAHOP_TRY(E.record(5));
    return E.record(6);
  }

  char* w = static_cast<char*>(ws);
  int32_t* idx = pb.off_idx != kNone ? reinterpret_cast<int32_t*>(w + pb.off_idx) : nullptr;
  const int had = pb.route == ADAHOP_ROUTE_MXFP4 ? 0 : 32;
  uint8_t* ac = reinterpret_cast<uint8_t*>(w + pb.off_a_codes);
  uint8_t* as = reinterpret_cast<uint8_t*>(w + pb.off_a_scales);
  uint8_t* bc = reinterpret_cast<uint8_t*>(w + pb.off_b_codes);
  uint8_t* bs = reinterpret_cast<uint8_t*>(w + pb.off_b_scales);
  uint16_t* ll = pb.off_lhs_lines != kNone ? reinterpret_cast<uint16_t*>(w + pb.off_lhs_lines) : nullptr;
  uint16_t* rl = pb.off_rhs_lines != kNone ? reinterpret_cast<uint16_t*>(w + pb.off_rhs_lines) : nullptr;
  if (ctx) {
    // X's indices, packed residual and lines as the forward kept them (read only).
    uint8_t* c = const_cast<uint8_t*>(ctx->base);
    idx = P.ctx_off_idx != kNone ? reinterpret_cast<int32_t*>(c + P.ctx_off_idx) : nullptr;
    bc = c + P.ctx_off_codes;
    bs = c + P.ctx_off_scales;
    rl = P.ctx_off_lines != kNone ? reinterpret_cast<uint16_t*>(c + P.ctx_off_lines) : nullptr;
  }
  const bool scan_lhs = pb.scan_tensor == 0;
  auto foid = [&](hipStream_t st, const QuantBeside* beside = nullptr, bool* beside_done = nullptr) {
    return foid_launch(scan_lhs ? lhs : rhs, scan_lhs ? s.lhs_rows : s.rhs_rows,
                       scan_lhs ? s.lhs_cols : s.rhs_cols, scan_lhs ? s.lhs_cols : s.rhs_cols,
                       pb.scan_axis, 64, pb.k, idx, P.off_foid != kNone ? w + P.off_foid : nullptr,
                       P.foid_bytes, st, beside, beside_done);
  };
  // With an outer outlier product the operand FOID does not scan is the
  // product's wide factor, read again in bf16 by the GEMM launch right after
  // its quantization. Up to a quarter of the 256 MB Infinity Cache, that
  // quantization keeps its source in the caches for it (o-proj BS 1 input
  // gradient, W 32 MB: -4 % per call, same-box A/B); larger factors would
  // not survive the other operand's pass and lose 0.2-2.4 % to the slower
  // loads. Every other quantization streams its source.
  const bool outer_oe = pb.route == ADAHOP_ROUTE_OE_LEFT || pb.route == ADAHOP_ROUTE_OE_RIGHT;
  const int64_t wide_bytes = 2 * (scan_lhs ? s.rhs_rows * s.rhs_cols : s.lhs_rows * s.lhs_cols);
  const bool keep_wide = outer_oe && wide_bytes <= (int64_t)64 << 20;
  const bool keep_lhs = keep_wide && !scan_lhs, keep_rhs = keep_wide && scan_lhs;
  auto quant_lhs = [&](hipStream_t st) {
    return iht_quant_launch(lhs, s.lhs_rows, s.lhs_cols, s.lhs_cols, s.lhs_contract, had,
                            P.zero_lhs ? idx : nullptr, P.zero_lhs ? pb.k : 0, P.lhs_zero_axis,
                            ac, as, ll, pb.layout, st, !keep_lhs);
  };
  auto quant_rhs = [&](hipStream_t st) {
    return iht_quant_launch(rhs, s.rhs_rows, s.rhs_cols, s.rhs_cols, s.rhs_contract, had,
                            P.zero_rhs ? idx : nullptr, P.zero_rhs ? pb.k : 0, P.rhs_zero_axis,
                            bc, bs, rl, pb.layout, st, !keep_rhs);
  };
  if (P.fused_groups > 0) {
    // One read of the operand FOID does not scan: FOID, the scanned
    // operand's quantization (which gathers the lines), then the other
    // operand's quantization forming the outlier product's partial sums,
    // their sum in order, and the GEMM, whose epilogue adds that sum to the
    // extracted lines. Stage events: after FOID, the lhs and rhs
    // quantizations in their order (with OE_RIGHT the lhs, quantized after
    // the rhs, falls in the outlier product's stage), the outlier product's
    // sum, the GEMM.
    float* partials = reinterpret_cast<float*>(w + P.off_partials);
    ADAHOP_TRY(foid(stream));
    ADAHOP_TRY(E.record(1));
    if (scan_lhs) {
      ADAHOP_TRY(quant_lhs(stream));
      ADAHOP_TRY(E.record(2));
      ADAHOP_TRY(iht_quant_oe_launch(rhs, s.rhs_rows, s.rhs_cols, s.rhs_cols, bc, bs, pb.layout, ll,
                                     pb.k, 1, partials, stream));
      ADAHOP_TRY(E.record(3));
    } else {
      ADAHOP_TRY(E.record(2));
      ADAHOP_TRY(quant_rhs(stream));
      ADAHOP_TRY(E.record(3));
      ADAHOP_TRY(iht_quant_oe_launch(lhs, s.lhs_rows, s.lhs_cols, s.lhs_cols, ac, as, pb.layout, rl,
                                     pb.k, 0, partials, stream));
    }
    ADAHOP_TRY(oe_reduce_launch(partials, P.fused_groups, (int64_t)pb.k * (scan_lhs ? s.n : s.m),
                                stream));
    ADAHOP_TRY(E.record(4));
    void* gemm_scratch = P.off_gemm != kNone ? w + P.off_gemm : nullptr;
    if (pb.layout == ADAHOP_LAYOUT_ROWS)
      ADAHOP_TRY(gemm_mx_stage_scales(ac, as, bc, bs, s.m, s.n, s.K, gemm_scratch, P.gemm_bytes, stream));
    OeEpilogue oe{};
    oe.mode = pb.route;
    oe.k = pb.k;
    oe.idx = idx;
    oe.partials = partials;
    oe.splits = P.fused_groups;
    ADAHOP_TRY(gemm_mx_launch(ac, as, bc, bs, s.m, s.n, s.K, pb.layout, oe, out, s.n, out_f32,
                              gemm_scratch, P.gemm_bytes, stream, E.at(5)));
    return E.record(6);
  }
  // OE_LEFT / OE_RIGHT zero lines of the scanned operand only, and only the
  // GEMM reads the other operand's packed form, so that operand's
  // quantization can run beside FOID. When FOID's selection fits one launch
  // (k <= 256, at most two levels), the two share FOID's launch (QuantBeside,
  // with the quantizer tiles of that operand's direction). Otherwise, with
  // large operands,
  // that operand is quantized on the side stream while FOID, the scanned
  // operand's quantization and the outlier product run on the caller's
  // stream; the join comes right before the GEMM (and the ROWS-layout scale
  // reordering).
  QuantBeside qb{};
  bool beside = false;
  if (!ctx && idx) {
    const bool other_lhs = !scan_lhs;
    if (had == 32 && (other_lhs ? !P.zero_lhs : !P.zero_rhs)) {
      const int64_t orows = other_lhs ? s.lhs_rows : s.rhs_rows, ocols = other_lhs ? s.lhs_cols : s.rhs_cols;
      qb.contract = other_lhs ? s.lhs_contract : s.rhs_contract;
      qb.src = other_lhs ? lhs : rhs;
      qb.K = qb.contract == ADAHOP_AXIS_ROWS ? orows : ocols;
      qb.outer = qb.contract == ADAHOP_AXIS_ROWS ? ocols : orows;
      qb.ld = ocols;
      qb.codes = other_lhs ? ac : bc;
      qb.scales = other_lhs ? as : bs;
      qb.layout = pb.layout;
      qb.stream_src = other_lhs ? !keep_lhs : !keep_rhs;
      const int64_t rows = scan_lhs ? s.lhs_rows : s.rhs_rows, cols = scan_lhs ? s.lhs_cols : s.rhs_cols;
      beside = foid_beside_fits(pb.scan_axis == ADAHOP_AXIS_ROWS ? rows : cols, pb.k, qb);
    }
  }
  SideJoin sj;
  SideStream* side = nullptr;
  if (ctx) {
    // Only the lhs is left to quantize: FOID and the rhs came with the context.
    ADAHOP_TRY(E.record(1));
    ADAHOP_TRY(quant_lhs(stream));
    ADAHOP_TRY(E.record(2));
  } else if (!beside && idx && (scan_lhs ? !P.zero_rhs : !P.zero_lhs) &&
             2 * (s.lhs_rows * s.lhs_cols + s.rhs_rows * s.rhs_cols) > ((int64_t)96 << 20)) {
    // The fork and the join cost ~15 us; they pay off only when the two
    // operands together exceed 96 MB of bf16 (same-box A/B, per call: o-proj
    // BS 1 input and weight gradients -2.4 % without the second stream, BS 2
    // input gradient -1.5 %; BS 2 weight gradient and from BS 4 on, faster
    // with it). The shared launch, where it applies, beats the second stream
    // too (same-box A/B: o-proj BS 2 weight gradient -5.8 %, BS 4 input and
    // weight gradients -2.6 % and -4.3 %, BS 8 weight gradient -1.6 %, the
    // down-proj weight gradient even) and one stream without it (o-proj BS 1
    // input and weight gradients -9.1 % and -7.4 %, BS 2 input gradient
    // -4.3 %).
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
      sj.lock = std::unique_lock<std::mutex>(g_side[dev].mu);
      side = side_stream_locked(dev);
      if (!side) sj.lock.unlock();
    }
  }
  if (side) {
    // Forked before FOID: FOID (latency-bound, few workgroups) runs beside
    // the other operand's quantization, and the scanned operand's
    // quantization after it overlaps that quantization's tail.
    ADAHOP_TRY(hip_ok(hipEventRecord(side->fork, stream), "hipEventRecord"));
    ADAHOP_TRY(hip_ok(hipStreamWaitEvent(side->stream, side->fork, 0), "hipStreamWaitEvent"));
    // From here on the join is owed, on every path.
    sj.side = side;
    sj.stream = stream;
    ADAHOP_TRY(scan_lhs ? quant_rhs(side->stream) : quant_lhs(side->stream));
    ADAHOP_TRY(foid(stream));
    ADAHOP_TRY(E.record(1));
    // The other operand's stage is empty on this stream.
    if (scan_lhs) {
      ADAHOP_TRY(quant_lhs(stream));
      ADAHOP_TRY(E.record(2));
      ADAHOP_TRY(E.record(3));
    } else {
      ADAHOP_TRY(E.record(2));
      ADAHOP_TRY(quant_rhs(stream));
      ADAHOP_TRY(E.record(3));
    }
  } else if (!ctx) {
    // One stream. With the shared launch the other operand's stage is empty.
    bool other_done = false;
    if (idx) ADAHOP_TRY(foid(stream, beside ? &qb : nullptr, &other_done));
    ADAHOP_TRY(E.record(1));
    if (!(other_done && !scan_lhs)) ADAHOP_TRY(quant_lhs(stream));
    ADAHOP_TRY(E.record(2));
    if (!(other_done && scan_lhs)) ADAHOP_TRY(quant_rhs(stream));
  }
  void* gemm_scratch = P.off_gemm != kNone ? w + P.off_gemm : nullptr;
  if (!side) {
    if (pb.layout == ADAHOP_LAYOUT_ROWS)
      ADAHOP_TRY(gemm_mx_stage_scales(ac, as, bc, bs, s.m, s.n, s.K, gemm_scratch, P.gemm_bytes, stream));
    ADAHOP_TRY(E.record(3));
  }

  OeEpilogue oe{};
  oe.mode = 0;
  if (pb.route == ADAHOP_ROUTE_OE_LEFT || pb.route == ADAHOP_ROUTE_OE_RIGHT) {
    float* partials = reinterpret_cast<float*>(w + P.off_partials);
    Bf16View X, Y;
    oe_views(P, lhs, rhs, ll, rl, &X, &Y);
    const int64_t nx = pb.route == ADAHOP_ROUTE_OE_LEFT ? pb.k : s.m;
    const int64_t ny = pb.route == ADAHOP_ROUTE_OE_LEFT ? s.n : pb.k;
    oe.mode = pb.route;
    oe.k = pb.k;
    oe.idx = idx;
    oe.a = X;
    oe.b = Y;
    // Inside the GEMM launch when the main kernel runs and the factors
    // allow it; else as its own kernels, before the GEMM.
    oe.fused_parts = gemm_mx_ring_used(ac, as, bc, bs, s.m, s.n, s.K, pb.layout)
                         ? oe_fused_parts(s.m, s.n, s.K, pb.route, pb.k, X, Y, true)
                         : 0;
    if (oe.fused_parts > 0) {
      oe.fused_ws = partials;
    } else {
      ADAHOP_TRY(oe_product_launch(X, Y, nx, ny, s.K, P.splits, partials, stream));
      oe.partials = partials;
      oe.splits = P.splits;
    }
  } else if (pb.route == ADAHOP_ROUTE_OE_INNER) {
    oe.mode = ADAHOP_ROUTE_OE_INNER;
    oe.k = pb.k;
    oe.a = lines_by_position(ll, line_len(s, true, P.lhs_zero_axis));  // (i, p)
    oe.b = lines_by_position(rl, line_len(s, false, P.rhs_zero_axis)); // (j, p)
  }
  ADAHOP_TRY(E.record(4));
  if (side) {
    ADAHOP_TRY(sj.join());
    sj.lock.unlock();
    if (pb.layout == ADAHOP_LAYOUT_ROWS)
      ADAHOP_TRY(gemm_mx_stage_scales(ac, as, bc, bs, s.m, s.n, s.K, gemm_scratch, P.gemm_bytes, stream));
  }
  ADAHOP_TRY(gemm_mx_launch(ac, as, bc, bs, s.m, s.n, s.K, pb.layout, oe, out, s.n, out_f32,
                            gemm_scratch, P.gemm_bytes, stream, E.at(5)));
  return E.record(6);
}

// Workspace of adahop_gemm_mx: the outlier product's partial sums (OE_LEFT,
// OE_RIGHT) first, then the GEMM's own scratch.
size_t gemm_mx_partials_bytes(int64_t m, int64_t n, int64_t K, const adahop_oe* oe) {
  if (!oe || (oe->route != ADAHOP_ROUTE_OE_LEFT && oe->route != ADAHOP_ROUTE_OE_RIGHT)) return 0;
  if (oe->k < 1) return 0;
  const int64_t nx = oe->route == ADAHOP_ROUTE_OE_LEFT ? oe->k : m;
  const int64_t ny = oe->route == ADAHOP_ROUTE_OE_LEFT ? n : oe->k;
  size_t bytes = align_up(sizeof(float) * (size_t)(oe_splits(nx, ny, K) + 1) * (size_t)nx * (size_t)ny, kAlign);
  const Bf16View X{oe->a.ptr, oe->a.ld, oe->a.inner_contiguous};
  const Bf16View Y{oe->b.ptr, oe->b.ld, oe->b.inner_contiguous};
  const int fp = oe_fused_parts(m, n, K, oe->route, oe->k, X, Y, false);
  if (fp > 0) bytes = std::max(bytes, oe_fused_bytes(m, n, oe->route, oe->k, fp));
  return bytes;
}

}  // namespace
}  // namespace adahop

namespace adahop {
namespace {
adahop_status detect_checks(const uint16_t* t, int64_t rows, int64_t cols, int64_t ld,
                            adahop_axis axis, int32_t probe, int32_t k, int32_t* idx_out) {
  if (!t || !idx_out) return fail(ADAHOP_ERR_INVALID, "adahop_detect: null pointer");
  if (rows < 1 || cols < 1 || ld < cols) return fail(ADAHOP_ERR_INVALID, "adahop_detect: bad sizes");
  if (axis != ADAHOP_AXIS_ROWS && axis != ADAHOP_AXIS_COLS)
    return fail(ADAHOP_ERR_INVALID, "adahop_detect: bad axis");
  if (probe < 1) return fail(ADAHOP_ERR_INVALID, "adahop_detect: probe < 1");
  const int64_t ncand = axis == ADAHOP_AXIS_ROWS ? rows : cols;
  if (k < 1 || k > ncand) return fail(ADAHOP_ERR_INVALID, "adahop_detect: k outside [1, candidates]");
  if (k > kMaxK) return fail(ADAHOP_ERR_UNSUPPORTED, "adahop_detect: k above 1024");
  if (!foid_fits(ncand, k)) return fail(ADAHOP_ERR_UNSUPPORTED, "adahop_detect: too many candidates");
  return ADAHOP_OK;
}

// Scratch of adahop_detect_noalloc: FOID's survivor lists and counter, in
// one array per GPU that the library holds until the process ends. In host
// code `scratch` names a host-side stand-in, never the device memory: its
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

struct NoAllocScratch {
  std::mutex mu;
  void* ptr[kMaxDevices] = {};
};
NoAllocScratch g_noalloc;

// The current device's address of `scratch`, looked up on its first use with
// that device current.
adahop_status noalloc_scratch(void** out) {
  int dev = 0;
  ADAHOP_TRY(hip_ok(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices) return fail(ADAHOP_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> g(g_noalloc.mu);
  if (!g_noalloc.ptr[dev]) {
    void* p = nullptr;
    ADAHOP_TRY(hip_ok(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress"));
    if (!p) return fail(ADAHOP_ERR_HIP, "hipGetSymbolAddress returned no address");
    g_noalloc.ptr[dev] = p;
  }
  *out = g_noalloc.ptr[dev];
  return ADAHOP_OK;
}
}  // namespace
}  // namespace adahop

using namespace adahop;

extern "C" {

const char* adahop_status_string(int status) {
  switch (status) {
    case ADAHOP_OK: return "ok";
    case ADAHOP_ERR_INVALID: return "invalid argument";
    case ADAHOP_ERR_UNSUPPORTED: return "unsupported";
    case ADAHOP_ERR_WORKSPACE: return "workspace too small";
    case ADAHOP_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* adahop_last_error(void) { return g_last_error.c_str(); }

int adahop_version(void) { return 1; }

adahop_route_t adahop_route(adahop_op op, adahop_pattern pat_lhs, adahop_pattern pat_rhs) {
  OpShape s;
  if (!op_shape(op, 1, 1, 1, &s) || !valid_pattern(pat_lhs) || !valid_pattern(pat_rhs))
    return ADAHOP_ROUTE_AUTO;
  // Patterns of the textbook operands A and B.
  const adahop_pattern a = s.lhs_transposed ? transposed(pat_lhs) : pat_lhs;
  const adahop_pattern b = s.rhs_transposed ? transposed(pat_rhs) : pat_rhs;
  // Outlier lines along the outer dimension (A's rows, B's columns) are what
  // mixing along the inner dimension cannot spread.
  const bool a_outer = a == ADAHOP_PAT_ROW;
  const bool b_outer = b == ADAHOP_PAT_COL;
  if (a_outer && b_outer) return ADAHOP_ROUTE_BF16;
  if (a_outer) return ADAHOP_ROUTE_OE_LEFT;
  if (b_outer) return ADAHOP_ROUTE_OE_RIGHT;
  return ADAHOP_ROUTE_IHT;
}

size_t adahop_detect_workspace_size(int64_t rows, int64_t cols, adahop_axis axis, int32_t k) {
  if (rows < 1 || cols < 1 || k < 1) return 0;
  return foid_workspace_bytes(axis == ADAHOP_AXIS_ROWS ? rows : cols, k);
}

adahop_status adahop_detect(const uint16_t* t, int64_t rows, int64_t cols, int64_t ld,
                            adahop_axis axis, int32_t probe, int32_t k, int32_t* idx_out,
                            void* ws, size_t ws_bytes, void* stream) {
  set_error("");
  ADAHOP_TRY(detect_checks(t, rows, cols, ld, axis, probe, k, idx_out));
  return foid_launch(t, rows, cols, ld, axis, probe, k, idx_out, ws, ws_bytes,
                     static_cast<hipStream_t>(stream));
}

size_t adahop_detect_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

adahop_status adahop_detect_noalloc(const uint16_t* t, int64_t rows, int64_t cols, int64_t ld,
                                    adahop_axis axis, int32_t probe, int32_t k,
                                    int32_t* idx_out, void* stream) {
  set_error("");
  ADAHOP_TRY(detect_checks(t, rows, cols, ld, axis, probe, k, idx_out));
  const size_t need = foid_workspace_bytes(axis == ADAHOP_AXIS_ROWS ? rows : cols, k);
  if (need > kNoAllocScratchBytes)
    return fail(ADAHOP_ERR_UNSUPPORTED,
                "adahop_detect_noalloc: this selection needs " + std::to_string(need) +
                    " bytes of scratch, above the library's static " +
                    std::to_string(kNoAllocScratchBytes) + "; call adahop_detect with a workspace");
  void* ws = nullptr;
  if (need > 0) ADAHOP_TRY(noalloc_scratch(&ws));
  return foid_launch(t, rows, cols, ld, axis, probe, k, idx_out, ws, need,
                     static_cast<hipStream_t>(stream));
}

adahop_status adahop_line_scores(const uint16_t* t, int64_t rows, int64_t cols, int64_t ld,
                                 adahop_axis axis, int32_t probe, double* scores_out,
                                 void* stream) {
  set_error("");
  if (!t || !scores_out) return fail(ADAHOP_ERR_INVALID, "adahop_line_scores: null pointer");
  if (rows < 1 || cols < 1 || ld < cols)
    return fail(ADAHOP_ERR_INVALID, "adahop_line_scores: bad sizes");
  if (axis != ADAHOP_AXIS_ROWS && axis != ADAHOP_AXIS_COLS)
    return fail(ADAHOP_ERR_INVALID, "adahop_line_scores: bad axis");
  if (probe < 1) return fail(ADAHOP_ERR_INVALID, "adahop_line_scores: probe < 1");
  return line_scores_launch(t, rows, cols, ld, axis, probe, scores_out,
                            static_cast<hipStream_t>(stream));
}

adahop_pattern adahop_classify_pattern(const double* row_scores, int64_t rows,
                                       const double* col_scores, int64_t cols,
                                       double threshold) {
  if (!row_scores || !col_scores || rows < 1 || cols < 1) return ADAHOP_PAT_NONE;
  // max / lower median of one axis' scores
  auto ratio = [](const double* v, int64_t n) {
    std::vector<double> s(v, v + n);
    std::nth_element(s.begin(), s.begin() + (n - 1) / 2, s.end());
    const double med = s[(size_t)((n - 1) / 2)];
    const double mx = *std::max_element(v, v + n);
    if (med > 0.0) return mx / med;
    return mx > 0.0 ? std::numeric_limits<double>::infinity() : 1.0;
  };
  const double rr = ratio(row_scores, rows), rc = ratio(col_scores, cols);
  if ((rr > rc ? rr : rc) < threshold) return ADAHOP_PAT_NONE;
  return rr >= rc ? ADAHOP_PAT_ROW : ADAHOP_PAT_COL;
}

adahop_status adahop_iht_quant(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld,
                               adahop_axis contract, int32_t hadamard_block,
                               const int32_t* zero_idx, int32_t nzero, adahop_axis zero_axis,
                               uint8_t* codes, uint8_t* scales, uint16_t* gathered,
                               void* stream) {
  set_error("");
  if (!src || !codes || !scales) return fail(ADAHOP_ERR_INVALID, "adahop_iht_quant: null pointer");
  if (rows < 1 || cols < 1 || ld < cols) return fail(ADAHOP_ERR_INVALID, "adahop_iht_quant: bad sizes");
  if (contract != ADAHOP_AXIS_ROWS && contract != ADAHOP_AXIS_COLS)
    return fail(ADAHOP_ERR_INVALID, "adahop_iht_quant: bad contraction axis");
  const int64_t K = contract == ADAHOP_AXIS_COLS ? cols : rows;
  if (K % 32 != 0) return fail(ADAHOP_ERR_INVALID, "adahop_iht_quant: K % 32 != 0");
  if (hadamard_block != 0 && hadamard_block != 32)
    return fail(ADAHOP_ERR_INVALID, "adahop_iht_quant: hadamard_block must be 0 or 32");
  if (nzero < 0 || (nzero > 0 && !zero_idx))
    return fail(ADAHOP_ERR_INVALID, "adahop_iht_quant: bad zero list");
  if (nzero > kMaxK) return fail(ADAHOP_ERR_UNSUPPORTED, "adahop_iht_quant: more than 1024 lines");
  if (nzero > 0 && zero_axis != ADAHOP_AXIS_ROWS && zero_axis != ADAHOP_AXIS_COLS)
    return fail(ADAHOP_ERR_INVALID, "adahop_iht_quant: bad zero axis");
  // Blocks along rows are read 16 bytes at a time; blocks down columns one
  // element per lane. Codes are written 16 bytes (or 4 bytes) at a time.
  if (contract == ADAHOP_AXIS_COLS && (!aligned16(src) || ld % 8 != 0))
    return fail(ADAHOP_ERR_UNSUPPORTED, "adahop_iht_quant: rows must be 16-byte aligned");
  if (!aligned16(codes) || !aligned16(gathered))
    return fail(ADAHOP_ERR_UNSUPPORTED,
                "adahop_iht_quant: codes and gathered must be 16-byte aligned");
  return iht_quant_launch(src, rows, cols, ld, contract, hadamard_block, zero_idx, nzero,
                          zero_axis, codes, scales, gathered, ADAHOP_LAYOUT_ROWS,
                          static_cast<hipStream_t>(stream));
}

size_t adahop_gemm_mx_workspace_size(int64_t m, int64_t n, int64_t K, const adahop_oe* oe) {
  if (m < 1 || n < 1 || K < 1) return 0;
  return gemm_mx_partials_bytes(m, n, K, oe) + gemm_mx_scratch_bytes(m, n, K, ADAHOP_LAYOUT_ROWS);
}

adahop_status adahop_gemm_mx(const adahop_mx_operand* A, const adahop_mx_operand* B,
                             const adahop_oe* oe, void* C, int64_t ldc,
                             adahop_out_dtype out_dtype, void* ws, size_t ws_bytes,
                             void* stream) {
  set_error("");
  if (!A || !B || !C || !A->codes || !A->scales || !B->codes || !B->scales)
    return fail(ADAHOP_ERR_INVALID, "adahop_gemm_mx: null pointer");
  if (A->outer < 1 || B->outer < 1 || A->K != B->K || A->K < 32 || A->K % 32 != 0)
    return fail(ADAHOP_ERR_INVALID, "adahop_gemm_mx: bad sizes (K must match and be a multiple of 32)");
  if (ldc < B->outer) return fail(ADAHOP_ERR_INVALID, "adahop_gemm_mx: ldc < n");
  if (out_dtype != ADAHOP_OUT_BF16 && out_dtype != ADAHOP_OUT_F32)
    return fail(ADAHOP_ERR_INVALID, "adahop_gemm_mx: bad out_dtype");
  if (!aligned16(A->codes) || !aligned16(B->codes))
    return fail(ADAHOP_ERR_UNSUPPORTED, "adahop_gemm_mx: codes must be 16-byte aligned");
  const int64_t m = A->outer, n = B->outer, K = A->K;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t need = adahop_gemm_mx_workspace_size(m, n, K, oe);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(ADAHOP_ERR_WORKSPACE, "adahop_gemm_mx: workspace too small: need " +
                                          std::to_string(need) + " bytes");
  if (need > 0 && !aligned16(ws))
    return fail(ADAHOP_ERR_UNSUPPORTED, "adahop_gemm_mx: the workspace must be 16-byte aligned");
  if (!gemm_mx_fits(m, n)) return fail(ADAHOP_ERR_UNSUPPORTED, "adahop_gemm_mx: too many output tiles");
  // Every check of the outlier descriptor comes before the first launch.
  OeEpilogue e{};
  int64_t oe_nx = 0, oe_ny = 0;
  if (oe) {
    if (oe->route != ADAHOP_ROUTE_OE_LEFT && oe->route != ADAHOP_ROUTE_OE_RIGHT &&
        oe->route != ADAHOP_ROUTE_OE_INNER)
      return fail(ADAHOP_ERR_INVALID, "adahop_gemm_mx: outlier route must be OE_LEFT, OE_RIGHT or OE_INNER");
    if (oe->k < 1 || !oe->a.ptr || !oe->b.ptr)
      return fail(ADAHOP_ERR_INVALID, "adahop_gemm_mx: bad outlier descriptor");
    if (oe->k > kMaxK) return fail(ADAHOP_ERR_UNSUPPORTED, "adahop_gemm_mx: k above 1024");
    if (oe->a.ld < 1 || oe->b.ld < 1)
      return fail(ADAHOP_ERR_INVALID, "adahop_gemm_mx: outlier views need ld >= 1");
    const Bf16View X{oe->a.ptr, oe->a.ld, oe->a.inner_contiguous};
    const Bf16View Y{oe->b.ptr, oe->b.ld, oe->b.inner_contiguous};
    if (oe->route == ADAHOP_ROUTE_OE_LEFT || oe->route == ADAHOP_ROUTE_OE_RIGHT) {
      if (!oe->idx) return fail(ADAHOP_ERR_INVALID, "adahop_gemm_mx: null idx");
      if (oe->k > (oe->route == ADAHOP_ROUTE_OE_LEFT ? m : n))
        return fail(ADAHOP_ERR_INVALID, "adahop_gemm_mx: k above the number of lines");
      oe_nx = oe->route == ADAHOP_ROUTE_OE_LEFT ? oe->k : m;
      oe_ny = oe->route == ADAHOP_ROUTE_OE_LEFT ? n : oe->k;
      if (!oe_product_fits(oe_nx, oe_ny))
        return fail(ADAHOP_ERR_UNSUPPORTED, "adahop_gemm_mx: outlier product too wide");
      e.mode = oe->route;
      e.k = oe->k;
      e.idx = oe->idx;
      e.partials = static_cast<const float*>(ws);
      e.splits = oe_splits(oe_nx, oe_ny, K);
      e.a = X;
      e.b = Y;
    } else {
      e.mode = ADAHOP_ROUTE_OE_INNER;
      e.k = oe->k;
      e.a = X;
      e.b = Y;
    }
  }
  const size_t partial_bytes = gemm_mx_partials_bytes(m, n, K, oe);
  void* scratch = need > partial_bytes ? static_cast<char*>(ws) + partial_bytes : nullptr;
  if (e.mode == ADAHOP_ROUTE_OE_LEFT || e.mode == ADAHOP_ROUTE_OE_RIGHT) {
    e.fused_parts = gemm_mx_ring_used(A->codes, A->scales, B->codes, B->scales, m, n, K, ADAHOP_LAYOUT_ROWS)
                        ? oe_fused_parts(m, n, K, e.mode, e.k, e.a, e.b, true)
                        : 0;
    if (e.fused_parts > 0) {
      e.fused_ws = static_cast<float*>(ws);
      e.partials = nullptr;
    }
  }
  ADAHOP_TRY(gemm_mx_stage_scales(A->codes, A->scales, B->codes, B->scales, m, n, K, scratch,
                                  need - partial_bytes, st));
  if ((e.mode == ADAHOP_ROUTE_OE_LEFT || e.mode == ADAHOP_ROUTE_OE_RIGHT) && e.fused_parts == 0)
    ADAHOP_TRY(oe_product_launch(e.a, e.b, oe_nx, oe_ny, K, e.splits, static_cast<float*>(ws), st));
  return gemm_mx_launch(A->codes, A->scales, B->codes, B->scales, m, n, K, ADAHOP_LAYOUT_ROWS, e,
                        C, ldc,
                        out_dtype == ADAHOP_OUT_F32 ? 1 : 0, scratch, need - partial_bytes, st);
}

adahop_status adahop_gemm_plan(adahop_op op, int64_t T, int64_t Din, int64_t Dout,
                               adahop_pattern pat_lhs, adahop_pattern pat_rhs,
                               adahop_route_t route, int32_t oe_rank, adahop_plan* plan) {
  set_error("");
  if (!plan) return fail(ADAHOP_ERR_INVALID, "adahop_gemm_plan: null plan");
  Plan P;
  ADAHOP_TRY(make_plan(op, T, Din, Dout, pat_lhs, pat_rhs, route, oe_rank, &P));
  *plan = P.pub;
  return ADAHOP_OK;
}

size_t adahop_gemm_workspace_size(adahop_op op, int64_t T, int64_t Din, int64_t Dout,
                                  adahop_pattern pat_lhs, adahop_pattern pat_rhs,
                                  adahop_route_t route, int32_t oe_rank) {
  Plan P;
  if (make_plan(op, T, Din, Dout, pat_lhs, pat_rhs, route, oe_rank, &P) != ADAHOP_OK) return 0;
  return P.pub.ws_bytes;
}

adahop_status adahop_gemm(adahop_op op, const uint16_t* lhs, const uint16_t* rhs, int64_t T,
                          int64_t Din, int64_t Dout, adahop_pattern pat_lhs,
                          adahop_pattern pat_rhs, adahop_route_t route, int32_t oe_rank,
                          void* out, adahop_out_dtype out_dtype, void* ws, size_t ws_bytes,
                          void* stream) {
  return run_gemm(op, lhs, rhs, T, Din, Dout, pat_lhs, pat_rhs, route, oe_rank, out, out_dtype,
                  ws, ws_bytes, static_cast<hipStream_t>(stream), nullptr);
}

adahop_status adahop_ctx_plan(int64_t T, int64_t Din, int64_t Dout, adahop_pattern pat_gy,
                              adahop_pattern pat_x, adahop_route_t route, int32_t oe_rank,
                              adahop_ctx_plan_t* plan) {
  set_error("");
  if (!plan) return fail(ADAHOP_ERR_INVALID, "adahop_ctx_plan: null plan");
  Plan P;
  ADAHOP_TRY(make_plan(ADAHOP_OP_WGRAD, T, Din, Dout, pat_gy, pat_x, route, oe_rank, &P, true));
  std::memset(plan, 0, sizeof(*plan));
  plan->route = P.pub.route;
  plan->T = T; plan->Din = Din; plan->Dout = Dout;
  plan->k = P.pub.k;
  plan->layout = P.pub.layout;
  plan->ctx_bytes = P.ctx_bytes;
  plan->off_idx = P.ctx_off_idx;
  plan->off_codes = P.ctx_off_codes;
  plan->off_scales = P.ctx_off_scales;
  plan->off_lines = P.ctx_off_lines;
  plan->save_ws_bytes = P.foid_bytes;
  plan->wgrad_ws_bytes = P.pub.ws_bytes;
  return ADAHOP_OK;
}

adahop_status adahop_ctx_save(const uint16_t* X, int64_t T, int64_t Din, int64_t Dout,
                              adahop_pattern pat_gy, adahop_pattern pat_x, adahop_route_t route,
                              int32_t oe_rank, void* ctx, size_t ctx_bytes, void* ws,
                              size_t ws_bytes, void* stream) {
  set_error("");
  if (!X || !ctx) return fail(ADAHOP_ERR_INVALID, "adahop_ctx_save: null X or context");
  Plan P;
  ADAHOP_TRY(make_plan(ADAHOP_OP_WGRAD, T, Din, Dout, pat_gy, pat_x, route, oe_rank, &P, true));
  if (ctx_bytes < P.ctx_bytes)
    return fail(ADAHOP_ERR_INVALID, "adahop_ctx_save: the context needs " +
                                        std::to_string(P.ctx_bytes) + " bytes");
  if (reinterpret_cast<uintptr_t>(ctx) & 15u)
    return fail(ADAHOP_ERR_UNSUPPORTED, "adahop_ctx_save: the context must be 16-byte aligned");
  if (P.foid_bytes > 0 && (!ws || ws_bytes < P.foid_bytes))
    return fail(ADAHOP_ERR_WORKSPACE, "adahop_ctx_save: workspace too small: need " +
                                          std::to_string(P.foid_bytes) + " bytes");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const adahop_plan& pb = P.pub;
  uint8_t* c = static_cast<uint8_t*>(ctx);
  int32_t* idx = P.ctx_off_idx != kNone ? reinterpret_cast<int32_t*>(c + P.ctx_off_idx) : nullptr;
  uint16_t* lines = P.ctx_off_lines != kNone ? reinterpret_cast<uint16_t*>(c + P.ctx_off_lines) : nullptr;
  // X [T, Din]: FOID over its columns (the weight gradient's OE-Right), then
  // the residual quantized along T (down the columns) with those columns
  // zeroed and copied out, in the layout the weight gradient's GEMM streams.
  if (idx)
    ADAHOP_TRY(foid_launch(X, T, Din, Din, ADAHOP_AXIS_COLS, 64, pb.k, idx, ws, P.foid_bytes, st));
  return iht_quant_launch(X, T, Din, Din, ADAHOP_AXIS_ROWS,
                          pb.route == ADAHOP_ROUTE_MXFP4 ? 0 : 32, idx, idx ? pb.k : 0,
                          ADAHOP_AXIS_COLS, c + P.ctx_off_codes, c + P.ctx_off_scales, lines,
                          pb.layout, st);
}

adahop_status adahop_gemm_wgrad_ctx(const uint16_t* GY, const void* ctx, size_t ctx_bytes,
                                    int64_t T, int64_t Din, int64_t Dout, adahop_pattern pat_gy,
                                    adahop_pattern pat_x, adahop_route_t route, int32_t oe_rank,
                                    void* out, adahop_out_dtype out_dtype, void* ws,
                                    size_t ws_bytes, void* stream, void* const* stage_events) {
  if (!ctx) {
    set_error("");
    return fail(ADAHOP_ERR_INVALID, "adahop_gemm_wgrad_ctx: null context");
  }
  const CtxIn in{static_cast<const uint8_t*>(ctx), ctx_bytes};
  return run_gemm(ADAHOP_OP_WGRAD, GY, nullptr, T, Din, Dout, pat_gy, pat_x, route, oe_rank, out,
                  out_dtype, ws, ws_bytes, static_cast<hipStream_t>(stream), stage_events, &in);
}

// Options of the _ex calls: NULL means all defaults; unknown (reserved)
// fields must be zero.
static adahop_status read_options(const adahop_gemm_options* opts, bool* oe_in_quant) {
  *oe_in_quant = false;
  if (!opts) return ADAHOP_OK;
  if (opts->oe_in_quant != 0 && opts->oe_in_quant != 1)
    return fail(ADAHOP_ERR_INVALID, "adahop_gemm_options: oe_in_quant must be 0 or 1");
  for (int32_t r : opts->reserved)
    if (r != 0) return fail(ADAHOP_ERR_INVALID, "adahop_gemm_options: reserved fields must be 0");
  *oe_in_quant = opts->oe_in_quant == 1;
  return ADAHOP_OK;
}

adahop_status adahop_gemm_plan_ex(adahop_op op, int64_t T, int64_t Din, int64_t Dout,
                                  adahop_pattern pat_lhs, adahop_pattern pat_rhs,
                                  adahop_route_t route, int32_t oe_rank,
                                  const adahop_gemm_options* opts, adahop_plan* plan) {
  set_error("");
  if (!plan) return fail(ADAHOP_ERR_INVALID, "adahop_gemm_plan_ex: null plan");
  bool oiq = false;
  ADAHOP_TRY(read_options(opts, &oiq));
  Plan P;
  ADAHOP_TRY(make_plan(op, T, Din, Dout, pat_lhs, pat_rhs, route, oe_rank, &P, false, oiq));
  *plan = P.pub;
  return ADAHOP_OK;
}

adahop_status adahop_gemm_ex(adahop_op op, const uint16_t* lhs, const uint16_t* rhs, int64_t T,
                             int64_t Din, int64_t Dout, adahop_pattern pat_lhs,
                             adahop_pattern pat_rhs, adahop_route_t route, int32_t oe_rank,
                             const adahop_gemm_options* opts, void* out,
                             adahop_out_dtype out_dtype, void* ws, size_t ws_bytes, void* stream,
                             void* const* stage_events) {
  set_error("");
  bool oiq = false;
  ADAHOP_TRY(read_options(opts, &oiq));
  return run_gemm(op, lhs, rhs, T, Din, Dout, pat_lhs, pat_rhs, route, oe_rank, out, out_dtype,
                  ws, ws_bytes, static_cast<hipStream_t>(stream), stage_events, nullptr, oiq);
}

adahop_status adahop_gemm_timed(adahop_op op, const uint16_t* lhs, const uint16_t* rhs,
                                int64_t T, int64_t Din, int64_t Dout, adahop_pattern pat_lhs,
                                adahop_pattern pat_rhs, adahop_route_t route, int32_t oe_rank,
                                void* out, adahop_out_dtype out_dtype, void* ws,
                                size_t ws_bytes, void* stream, void* const* stage_events) {
  return run_gemm(op, lhs, rhs, T, Din, Dout, pat_lhs, pat_rhs, route, oe_rank, out, out_dtype,
                  ws, ws_bytes, static_cast<hipStream_t>(stream), stage_events);
}

}  // extern "C"
