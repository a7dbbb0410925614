"""Python binding of the AdaHOP GEMM library (libadahop.so, HIP for gfx950).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch supplies device memory and the current stream. The functions
carry the C ABI's names (see include/adahop.h for the contract of each).

bf16 tensors may be passed as torch.bfloat16 or as int16 bit patterns.
There is no CPU fallback: if the library is missing this module raises.
"""
import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libadahop.so")

PAT = {"N": 0, "R": 1, "C": 2}
OP = {"FWD": 0, "DGRAD": 1, "WGRAD": 2}
ROUTE = {"AUTO": -1, "BF16": 0, "IHT": 1, "OE_LEFT": 2, "OE_RIGHT": 3, "OE_INNER": 4, "MXFP4": 5}
ROUTE_NAME = {v: k for k, v in ROUTE.items()}
AXIS = {"ROWS": 0, "COLS": 1}
OUT = {torch.bfloat16: 0, torch.float32: 1}
STAGE_EVENTS = 7
STAGES = ("foid", "quant_lhs", "quant_rhs", "oe_product", "gemm", "gemm_tail")

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_int = ctypes.c_int
_sz = ctypes.c_size_t


class AdahopError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"adahop status {status}: {detail}")


class MxOperand(ctypes.Structure):
    _fields_ = [("codes", _p), ("scales", _p), ("outer", _i64), ("K", _i64)]


class Bf16View(ctypes.Structure):
    _fields_ = [("ptr", _p), ("ld", _i64), ("inner_contiguous", _i32), ("reserved", _i32)]


class OeDesc(ctypes.Structure):
    _fields_ = [("route", _int), ("k", _i32), ("idx", _p), ("a", Bf16View), ("b", Bf16View)]


class Plan(ctypes.Structure):
    _fields_ = [("route", _int), ("m", _i64), ("n", _i64), ("K", _i64), ("k", _i32),
                ("scan_tensor", _i32), ("scan_axis", _int), ("layout", _int),
                ("ws_bytes", _sz), ("off_idx", _sz), ("off_a_codes", _sz),
                ("off_a_scales", _sz), ("off_b_codes", _sz), ("off_b_scales", _sz),
                ("off_lhs_lines", _sz), ("off_rhs_lines", _sz), ("oe_in_quant", _i32)]


class GemmOptions(ctypes.Structure):
    _fields_ = [("oe_in_quant", _i32), ("reserved", _i32 * 7)]


class CtxPlan(ctypes.Structure):
    _fields_ = [("route", _int), ("T", _i64), ("Din", _i64), ("Dout", _i64), ("k", _i32),
                ("layout", _int), ("ctx_bytes", _sz), ("off_idx", _sz), ("off_codes", _sz),
                ("off_scales", _sz), ("off_lines", _sz), ("save_ws_bytes", _sz),
                ("wgrad_ws_bytes", _sz)]


# Exported symbols and their C signatures (argtypes, restype).
SIGNATURES = {
    "adahop_status_string": ([_int], ctypes.c_char_p),
    "adahop_last_error": ([], ctypes.c_char_p),
    "adahop_version": ([], _int),
    "adahop_route": ([_int, _int, _int], _int),
    "adahop_detect_workspace_size": ([_i64, _i64, _int, _i32], _sz),
    "adahop_detect": ([_p, _i64, _i64, _i64, _int, _i32, _i32, _p, _p, _sz, _p], _int),
    "adahop_detect_noalloc_max_bytes": ([], _sz),
    "adahop_detect_noalloc": ([_p, _i64, _i64, _i64, _int, _i32, _i32, _p, _p], _int),
    "adahop_line_scores": ([_p, _i64, _i64, _i64, _int, _i32, _p, _p], _int),
    "adahop_classify_pattern": ([ctypes.POINTER(ctypes.c_double), _i64,
                                 ctypes.POINTER(ctypes.c_double), _i64, ctypes.c_double], _int),
    "adahop_iht_quant": ([_p, _i64, _i64, _i64, _int, _i32, _p, _i32, _int, _p, _p, _p, _p],
                         _int),
    "adahop_gemm_mx_workspace_size": ([_i64, _i64, _i64, ctypes.POINTER(OeDesc)], _sz),
    "adahop_gemm_mx": ([ctypes.POINTER(MxOperand), ctypes.POINTER(MxOperand),
                        ctypes.POINTER(OeDesc), _p, _i64, _int, _p, _sz, _p], _int),
    "adahop_gemm_plan": ([_int, _i64, _i64, _i64, _int, _int, _int, _i32,
                          ctypes.POINTER(Plan)], _int),
    "adahop_gemm_workspace_size": ([_int, _i64, _i64, _i64, _int, _int, _int, _i32], _sz),
    "adahop_gemm": ([_int, _p, _p, _i64, _i64, _i64, _int, _int, _int, _i32, _p, _int, _p,
                     _sz, _p], _int),
    "adahop_gemm_timed": ([_int, _p, _p, _i64, _i64, _i64, _int, _int, _int, _i32, _p, _int,
                           _p, _sz, _p, _p], _int),
    "adahop_gemm_plan_ex": ([_int, _i64, _i64, _i64, _int, _int, _int, _i32,
                             ctypes.POINTER(GemmOptions), ctypes.POINTER(Plan)], _int),
    "adahop_gemm_ex": ([_int, _p, _p, _i64, _i64, _i64, _int, _int, _int, _i32,
                        ctypes.POINTER(GemmOptions), _p, _int, _p, _sz, _p, _p], _int),
    "adahop_ctx_plan": ([_i64, _i64, _i64, _int, _int, _int, _i32, ctypes.POINTER(CtxPlan)], _int),
    "adahop_ctx_save": ([_p, _i64, _i64, _i64, _int, _int, _int, _i32, _p, _sz, _p, _sz, _p],
                        _int),
    "adahop_gemm_wgrad_ctx": ([_p, _p, _sz, _i64, _i64, _i64, _int, _int, _int, _i32, _p, _int,
                               _p, _sz, _p, _p], _int),
}

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "python -c 'import __graft_entry__ as g; g.build()'")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def _check(status: int):
    if status != 0:
        raise AdahopError(status, lib().adahop_last_error().decode())


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _bf16_ptr(t: torch.Tensor, name: str) -> int:
    if t.dtype not in (torch.bfloat16, torch.int16):
        raise TypeError(f"{name}: expected bfloat16 (or int16 bit patterns), got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name}: expected a 2-D tensor with unit column stride")
    return t.data_ptr()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _axis(a) -> int:
    return AXIS[a] if isinstance(a, str) else int(a)


def adahop_route(op: str, pat_lhs: str, pat_rhs: str) -> str:
    r = lib().adahop_route(OP[op], PAT[pat_lhs], PAT[pat_rhs])
    if r == ROUTE["AUTO"]:
        raise ValueError("invalid op or pattern")
    return ROUTE_NAME[r]


def adahop_detect_workspace_size(rows: int, cols: int, axis, k: int) -> int:
    return lib().adahop_detect_workspace_size(rows, cols, _axis(axis), k)


def adahop_detect(t: torch.Tensor, axis, k: int, probe: int = 64,
                  idx_out: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """FOID: int32 [k] indices of the outlier rows/columns of t, ascending."""
    ptr = _bf16_ptr(t, "t")
    rows, cols = t.shape
    if idx_out is None:
        idx_out = torch.empty(max(k, 1), dtype=torch.int32, device=t.device)
    need = adahop_detect_workspace_size(rows, cols, axis, k)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=t.device)
    _check(lib().adahop_detect(ptr, rows, cols, t.stride(0), _axis(axis), probe, k,
                               idx_out.data_ptr(), _ptr(ws), 0 if ws is None else ws.numel(),
                               _stream(t.device)))
    return idx_out[:k]


def adahop_detect_noalloc(t: torch.Tensor, axis, k: int, probe: int = 64,
                          idx_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """FOID with the library's static scratch (no workspace): int32 [k]
    indices, ascending. Pass idx_out to keep the call free of allocation."""
    ptr = _bf16_ptr(t, "t")
    rows, cols = t.shape
    if idx_out is None:
        idx_out = torch.empty(max(k, 1), dtype=torch.int32, device=t.device)
    _check(lib().adahop_detect_noalloc(ptr, rows, cols, t.stride(0), _axis(axis), probe, k,
                                       idx_out.data_ptr(), _stream(t.device)))
    return idx_out[:k]


def adahop_line_scores(t: torch.Tensor, axis, probe: int = 64,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """FOID's score of every row (axis ROWS) or column (COLS) of t: fp64 on the device."""
    ptr = _bf16_ptr(t, "t")
    rows, cols = t.shape
    n = rows if _axis(axis) == AXIS["ROWS"] else cols
    if out is None:
        out = torch.empty(n, dtype=torch.float64, device=t.device)
    _check(lib().adahop_line_scores(ptr, rows, cols, t.stride(0), _axis(axis), probe,
                                    out.data_ptr(), _stream(t.device)))
    return out


CLASSIFY_THRESHOLD = 8.0


def adahop_classify_pattern(row_scores, col_scores, threshold: float = CLASSIFY_THRESHOLD) -> str:
    """"R", "C" or "N" from a tensor's row and column scores (host copies are made)."""
    r = np.ascontiguousarray(torch.as_tensor(row_scores).detach().cpu().numpy(), dtype=np.float64)
    c = np.ascontiguousarray(torch.as_tensor(col_scores).detach().cpu().numpy(), dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    p = lib().adahop_classify_pattern(r.ctypes.data_as(dp), r.size, c.ctypes.data_as(dp), c.size,
                                      float(threshold))
    return {v: k for k, v in PAT.items()}[p]


def adahop_calibrate(t: torch.Tensor, probe: int = 64,
                     threshold: float = CLASSIFY_THRESHOLD) -> str:
    """The pattern of a bf16 tensor from its row and column scores."""
    rs = adahop_line_scores(t, "ROWS", probe)
    cs = adahop_line_scores(t, "COLS", probe)
    return adahop_classify_pattern(rs, cs, threshold)


def adahop_iht_quant(src: torch.Tensor, contract, hadamard_block: int = 32,
                     zero_idx: Optional[torch.Tensor] = None, zero_axis="ROWS",
                     gather: bool = True):
    """(codes [outer][K/2] u8, scales [outer][K/32] u8, gathered bf16 or None)."""
    ptr = _bf16_ptr(src, "src")
    rows, cols = src.shape
    c = _axis(contract)
    K, outer = (cols, rows) if c == AXIS["COLS"] else (rows, cols)
    dev = src.device
    codes = torch.empty((outer, max(K // 2, 1)), dtype=torch.uint8, device=dev)
    scales = torch.empty((outer, max(K // 32, 1)), dtype=torch.uint8, device=dev)
    nz = 0 if zero_idx is None else zero_idx.numel()
    za = _axis(zero_axis)
    gathered = None
    if nz and gather:
        shape = (nz, cols) if za == AXIS["ROWS"] else (nz, rows)   # one line per row
        gathered = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    if zero_idx is not None and zero_idx.dtype != torch.int32:
        raise TypeError("zero_idx must be int32")
    _check(lib().adahop_iht_quant(ptr, rows, cols, src.stride(0), c, hadamard_block,
                                  _ptr(zero_idx), nz, za, codes.data_ptr(), scales.data_ptr(),
                                  _ptr(gathered), _stream(dev)))
    return codes, scales, gathered


def bf16_view(t: torch.Tensor, inner_contiguous: bool) -> Bf16View:
    return Bf16View(_bf16_ptr(t, "view"), t.stride(0), int(inner_contiguous), 0)


def adahop_gemm_mx(a_codes, a_scales, b_codes, b_scales, oe: Optional[dict] = None,
                   out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None):
    """C = deq(A) deq(B)^T (+ the outlier term). oe: {"route", "k", "idx", "a":
    (tensor, inner_contiguous), "b": (tensor, inner_contiguous)}."""
    m, n, K = a_codes.shape[0], b_codes.shape[0], a_codes.shape[1] * 2
    A = MxOperand(a_codes.data_ptr(), a_scales.data_ptr(), m, K)
    B = MxOperand(b_codes.data_ptr(), b_scales.data_ptr(), n, b_codes.shape[1] * 2)
    dev = a_codes.device
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
    desc = None
    ws = None
    if oe is not None:
        idx = oe.get("idx")
        desc = OeDesc(ROUTE[oe["route"]], oe["k"], _ptr(idx), bf16_view(*oe["a"]),
                      bf16_view(*oe["b"]))
    need = lib().adahop_gemm_mx_workspace_size(
        m, n, K, ctypes.byref(desc) if desc is not None else None)
    if need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib().adahop_gemm_mx(ctypes.byref(A), ctypes.byref(B),
                                ctypes.byref(desc) if desc is not None else None,
                                out.data_ptr(), out.stride(0), OUT[out.dtype], _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(dev)))
    return out


def _options(oe_in_quant: bool):
    return GemmOptions(oe_in_quant=1 if oe_in_quant else 0)


def adahop_gemm_plan(op: str, T: int, Din: int, Dout: int, pat_lhs="N", pat_rhs="N",
                     route: Optional[str] = None, oe_rank: int = 64,
                     oe_in_quant: bool = False) -> Plan:
    """The call's plan; oe_in_quant asks for the outlier product formed in
    the other operand's quantization (adahop_gemm_plan_ex)."""
    p = Plan()
    if oe_in_quant:
        o = _options(True)
        _check(lib().adahop_gemm_plan_ex(OP[op], T, Din, Dout, PAT[pat_lhs], PAT[pat_rhs],
                                         ROUTE[route or "AUTO"], oe_rank, ctypes.byref(o),
                                         ctypes.byref(p)))
    else:
        _check(lib().adahop_gemm_plan(OP[op], T, Din, Dout, PAT[pat_lhs], PAT[pat_rhs],
                                      ROUTE[route or "AUTO"], oe_rank, ctypes.byref(p)))
    return p


def adahop_gemm_workspace_size(op: str, T: int, Din: int, Dout: int, pat_lhs="N",
                               pat_rhs="N", route: Optional[str] = None,
                               oe_rank: int = 64) -> int:
    return adahop_gemm_plan(op, T, Din, Dout, pat_lhs, pat_rhs, route, oe_rank).ws_bytes


def _gemm_dims(op, lhs, rhs):
    if op == "FWD":
        (T, Din), (Dout, Din2) = lhs.shape, rhs.shape
        ok = Din == Din2
        out_shape = (T, Dout)
    elif op == "DGRAD":
        (T, Dout), (Dout2, Din) = lhs.shape, rhs.shape
        ok = Dout == Dout2
        out_shape = (T, Din)
    elif op == "WGRAD":
        (T, Dout), (T2, Din) = lhs.shape, rhs.shape
        ok = T == T2
        out_shape = (Dout, Din)
    else:
        raise ValueError(f"invalid op {op}")
    if not ok:
        raise ValueError(f"{op}: operand shapes {tuple(lhs.shape)} and {tuple(rhs.shape)} disagree")
    return T, Din, Dout, out_shape


def adahop_gemm(op: str, lhs: torch.Tensor, rhs: torch.Tensor, pat_lhs="N", pat_rhs="N",
                route: Optional[str] = None, oe_rank: int = 64, out_dtype=torch.bfloat16,
                out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                stage_events: Optional[Sequence] = None, oe_in_quant: bool = False):
    """One AdaHOP product; returns the output tensor. `ws` (uint8, at least
    the planned size) is optional; after the call it holds the quantized
    operands at the offsets of adahop_gemm_plan. stage_events: STAGE_EVENTS
    torch.cuda.Event(enable_timing=True), recorded at the stage boundaries.
    oe_in_quant: form the outlier product in the other operand's
    quantization where it applies (adahop_gemm_ex)."""
    for t, nm in ((lhs, "lhs"), (rhs, "rhs")):
        _bf16_ptr(t, nm)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    T, Din, Dout, out_shape = _gemm_dims(op, lhs, rhs)
    plan = adahop_gemm_plan(op, T, Din, Dout, pat_lhs, pat_rhs, route, oe_rank, oe_in_quant)
    dev = lhs.device
    if out is None:
        out = torch.empty(out_shape, dtype=out_dtype, device=dev)
    if ws is None and plan.ws_bytes:
        ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device=dev)
    args = [OP[op], lhs.data_ptr(), rhs.data_ptr(), T, Din, Dout, PAT[pat_lhs], PAT[pat_rhs],
            ROUTE[route or "AUTO"], oe_rank, out.data_ptr(), OUT[out.dtype], _ptr(ws),
            0 if ws is None else ws.numel(), _stream(dev)]
    handles = None
    if stage_events is not None:
        if len(stage_events) != STAGE_EVENTS:
            raise ValueError(f"stage_events needs {STAGE_EVENTS} events")
        handles = (ctypes.c_void_p * STAGE_EVENTS)(*[_event_handle(e) for e in stage_events])
    if oe_in_quant:
        o = _options(True)
        _check(lib().adahop_gemm_ex(*args[:10], ctypes.byref(o), *args[10:], handles))
    elif handles is None:
        _check(lib().adahop_gemm(*args))
    else:
        _check(lib().adahop_gemm_timed(*args, handles))
    return out


def _event_handle(ev: "torch.cuda.Event") -> int:
    # torch creates the underlying hipEvent lazily, at the first record().
    if ev.cuda_event == 0:
        ev.record()
    return ev.cuda_event


LAYOUT_ROWS, LAYOUT_KCHUNK = 0, 1


def unpack_packed(codes: torch.Tensor, scales: torch.Tensor, outer: int, K: int, layout: int):
    """Packed operand bytes in `layout` as row-major ([outer][K/2] codes,
    [outer][K/32] scales); a K-chunked operand is reordered (a copy)."""
    if layout == LAYOUT_KCHUNK:     # [K/128][outer][64], [K/128][outer][4]
        codes = codes.view(K // 128, outer, 64).permute(1, 0, 2).reshape(outer, K // 2)
        # a chunk's scale bytes are its blocks' in the order 0, 2, 1, 3
        scales = scales.view(K // 128, outer, 4)[:, :, [0, 2, 1, 3]]
        scales = scales.permute(1, 0, 2).reshape(outer, K // 32)
    return codes.view(outer, K // 2), scales.view(outer, K // 32)


def workspace_views(ws: torch.Tensor, plan: Plan) -> dict:
    """The intermediates a call leaves in its workspace, as tensors. Packed
    operands are returned in the row-major layout ([outer][K/2] codes,
    [outer][K/32] scales); a K-chunked plan's are reordered into it (a copy)."""
    none = (1 << 64) - 1
    m, n, K, k = plan.m, plan.n, plan.K, plan.k

    def region(off, count, dtype):
        if off == none:
            return None
        nbytes = count * torch.tensor([], dtype=dtype).element_size()
        return ws[off:off + nbytes].view(dtype)

    def packed(off_codes, off_scales, outer):
        codes = region(off_codes, outer * (K // 2), torch.uint8)
        scales = region(off_scales, outer * (K // 32), torch.uint8)
        if codes is None:
            return None, None
        return unpack_packed(codes, scales, outer, K, plan.layout)

    out = {"idx": region(plan.off_idx, k, torch.int32)}
    out["a_codes"], out["a_scales"] = packed(plan.off_a_codes, plan.off_a_scales, m)
    out["b_codes"], out["b_scales"] = packed(plan.off_b_codes, plan.off_b_scales, n)
    return out


# ---------------------------------------------------------------------------
# Saved forward context of the activation X for the weight gradient
# ---------------------------------------------------------------------------
def adahop_ctx_plan(T: int, Din: int, Dout: int, pat_gy="N", pat_x="N",
                    route: Optional[str] = None, oe_rank: int = 64) -> CtxPlan:
    p = CtxPlan()
    _check(lib().adahop_ctx_plan(T, Din, Dout, PAT[pat_gy], PAT[pat_x], ROUTE[route or "AUTO"],
                                 oe_rank, ctypes.byref(p)))
    return p


def adahop_ctx_save(X: torch.Tensor, Dout: int, pat_gy="N", pat_x="N",
                    route: Optional[str] = None, oe_rank: int = 64,
                    ctx: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The context X [T, Din] keeps for its weight gradient (uint8 device
    buffer laid out as adahop_ctx_plan says)."""
    _bf16_ptr(X, "X")
    if not X.is_contiguous():
        raise ValueError("X must be contiguous")
    T, Din = X.shape
    plan = adahop_ctx_plan(T, Din, Dout, pat_gy, pat_x, route, oe_rank)
    if ctx is None:
        ctx = torch.empty(max(plan.ctx_bytes, 1), dtype=torch.uint8, device=X.device)
    if ws is None and plan.save_ws_bytes:
        ws = torch.empty(plan.save_ws_bytes, dtype=torch.uint8, device=X.device)
    _check(lib().adahop_ctx_save(X.data_ptr(), T, Din, Dout, PAT[pat_gy], PAT[pat_x],
                                 ROUTE[route or "AUTO"], oe_rank, ctx.data_ptr(), ctx.numel(),
                                 _ptr(ws), 0 if ws is None else ws.numel(), _stream(X.device)))
    return ctx


def adahop_gemm_wgrad_ctx(GY: torch.Tensor, ctx: torch.Tensor, Din: int, pat_gy="N", pat_x="N",
                          route: Optional[str] = None, oe_rank: int = 64,
                          out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None,
                          ws: Optional[torch.Tensor] = None,
                          stage_events: Optional[Sequence] = None) -> torch.Tensor:
    """dW [Dout, Din] = GY^T X with X taken from its saved context."""
    _bf16_ptr(GY, "GY")
    if not GY.is_contiguous():
        raise ValueError("GY must be contiguous")
    if ctx.dtype != torch.uint8 or not ctx.is_cuda:
        raise TypeError("ctx must be a uint8 device tensor")
    T, Dout = GY.shape
    plan = adahop_ctx_plan(T, Din, Dout, pat_gy, pat_x, route, oe_rank)
    if out is None:
        out = torch.empty((Dout, Din), dtype=out_dtype, device=GY.device)
    if ws is None and plan.wgrad_ws_bytes:
        ws = torch.empty(plan.wgrad_ws_bytes, dtype=torch.uint8, device=GY.device)
    handles = None
    if stage_events is not None:
        if len(stage_events) != STAGE_EVENTS:
            raise ValueError(f"stage_events needs {STAGE_EVENTS} events")
        handles = (ctypes.c_void_p * STAGE_EVENTS)(*[_event_handle(e) for e in stage_events])
    _check(lib().adahop_gemm_wgrad_ctx(GY.data_ptr(), ctx.data_ptr(), ctx.numel(), T, Din, Dout,
                                       PAT[pat_gy], PAT[pat_x], ROUTE[route or "AUTO"], oe_rank,
                                       out.data_ptr(), OUT[out.dtype], _ptr(ws),
                                       0 if ws is None else ws.numel(), _stream(GY.device),
                                       handles))
    return out


def ctx_views(ctx: torch.Tensor, plan: CtxPlan) -> dict:
    """The arrays of a saved context as tensors: idx [k] (or None), codes
    [Din][T/2] and scales [Din][T/32] row-major (reordered from K-chunked if
    needed), lines [k][T] bf16 bits (or None)."""
    none = (1 << 64) - 1
    T, Din, k = plan.T, plan.Din, plan.k
    codes = ctx[plan.off_codes:plan.off_codes + Din * T // 2]
    scales = ctx[plan.off_scales:plan.off_scales + Din * T // 32]
    c, sc = unpack_packed(codes, scales, Din, T, plan.layout)
    return {"idx": None if plan.off_idx == none else ctx[plan.off_idx:plan.off_idx + 4 * k].view(torch.int32),
            "codes": c, "scales": sc,
            "lines": None if plan.off_lines == none
            else ctx[plan.off_lines:plan.off_lines + 2 * k * T].view(torch.int16).view(k, T)}
