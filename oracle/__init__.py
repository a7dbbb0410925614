"""AdaHOP oracle: plain, slow CPU reference of the per-GEMM path.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package. The product path (the
GPU library and its binding) never loads it, and it never loads the product.

The arithmetic lives in ``adahop_ref.c`` (plain C11, fp64 where the method
leaves the precision open, the kernels' fp32 where floating point decides a
quantized code). This module only marshals numpy arrays into it; the
composition of the steps into one GEMM call is in ``pipeline.py``.

Parity unpinned: ``route`` beyond the products the pages configure (their
cells and Table 1's pair counts pin it; Fig. 5's table is not legible, so the
rest is the derivation stated in ``adahop_ref.c``). Every other function is
pinned by the CPU tests against closed forms, printed values or brute force.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_adahop.so")
_lib = None

# Enumerations (the oracle's own copy; the values match the public contract).
PAT = {"N": 0, "R": 1, "C": 2}
OP = {"FWD": 0, "DGRAD": 1, "WGRAD": 2}
ROUTE = {"BF16": 0, "IHT": 1, "OE_LEFT": 2, "OE_RIGHT": 3, "OE_INNER": 4, "MXFP4": 5}
ROUTE_NAME = {v: k for k, v in ROUTE.items()}
ROWS, COLS = 0, 1

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_int = ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: run python oracle/build.py")
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "adahop_ref_route": ([_int, _int, _int], _int),
        "adahop_ref_scan_target": ([_int, _int, _p, _p], _int),
        "adahop_ref_foid": ([_p, _i64, _i64, _i64, _int, _int, _int, _p, _p], _int),
        "adahop_ref_fwht32": ([_p], None),
        "adahop_ref_e2m1_magnitude": ([ctypes.c_double], _int),
        "adahop_ref_e2m1_value": ([_int], ctypes.c_double),
        "adahop_ref_mx_block": ([_p, _p, _p], None),
        "adahop_ref_iht_quant": ([_p, _i64, _i64, _i64, _int, _int, _p, _i32, _int, _p, _p, _p],
                                 _int),
        "adahop_ref_gemm_mx": ([_p, _p, _p, _p, _i64, _p, _i64, _p, _i64, _p, _p], _int),
        "adahop_ref_gemm_bf16": ([_p, _i64, _int, _p, _i64, _int, _i64, _p, _i64, _p, _i64,
                                  _p, _p], _int),
        "adahop_ref_walk_mx": ([_p, _p, _p, _p, _i64, _i64, _p, _i64, _p, _i64, _p, _p], _int),
        "adahop_ref_walk_bf16": ([_p, _i64, _int, _p, _i64, _int, _i64, _i64, _p, _i64, _p, _i64,
                                  _p, _p], _int),
        "adahop_ref_dequant": ([_p, _p, _i64, _i64, _p], _int),
        "adahop_ref_max_threads": ([], _int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


def max_threads() -> int:
    return _load().adahop_ref_max_threads()


def route(op: str, pat_lhs: str, pat_rhs: str) -> str:
    r = _load().adahop_ref_route(OP[op], PAT[pat_lhs], PAT[pat_rhs])
    _check(0 if r >= 0 else -1, "route")
    return ROUTE_NAME[r]


def scan_target(op: str, route_name: str):
    """(tensor, axis): tensor 0 = lhs, 1 = rhs; axis ROWS/COLS."""
    t, a = ctypes.c_int(), ctypes.c_int()
    _check(_load().adahop_ref_scan_target(OP[op], ROUTE[route_name], ctypes.byref(t),
                                          ctypes.byref(a)), "scan_target")
    return t.value, a.value


def foid(t: np.ndarray, axis: int, k: int, probe: int = 64, return_var: bool = False):
    assert t.dtype == np.uint16 and t.ndim == 2
    t = np.ascontiguousarray(t)
    rows, cols = t.shape
    idx = np.zeros(max(k, 1), dtype=np.int32)
    var = np.zeros(rows if axis == ROWS else cols, dtype=np.float64) if return_var else None
    _check(_load().adahop_ref_foid(_ptr(t), rows, cols, cols, axis, probe, k, _ptr(idx),
                                   _ptr(var)), "foid")
    return (idx[:k], var) if return_var else idx[:k]


def line_scores(t: np.ndarray, axis: int, probe: int = 64) -> np.ndarray:
    """FOID's score of every row (ROWS) or column (COLS) of t: the probe
    variance that FOID ranks (its var_out), fp64."""
    return foid(t, axis, 1, probe=probe, return_var=True)[1]


def classify_pattern(row_scores, col_scores, threshold: float) -> str:
    """Pattern of a tensor from its line scores: "R", "C" or "N".

    Table 1 of the AdaHOP pages names the patterns (a few outlier rows, a few
    outlier columns, or none) and Fig. 4 / Fig. 8 show them; the pages give
    no numeric test. Reading: per axis, r = largest score / lower median
    score (the element of rank (n - 1) // 2 in ascending order); "N" when the
    larger r is below the threshold, else "R" if r_rows >= r_cols, else "C".
    A zero median with a positive maximum is an infinite ratio; an all-zero
    axis has ratio 1.
    """
    def ratio(v):
        s = sorted(float(x) for x in v)
        med, top = s[(len(s) - 1) // 2], s[-1]
        if med > 0.0:
            return top / med
        return float("inf") if top > 0.0 else 1.0

    rr, rc = ratio(row_scores), ratio(col_scores)
    if max(rr, rc) < threshold:
        return "N"
    return "R" if rr >= rc else "C"


def fwht32(y: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32).copy()
    assert y.shape == (32,)
    _load().adahop_ref_fwht32(_ptr(y))
    return y


def e2m1_magnitude(v: float) -> int:
    return _load().adahop_ref_e2m1_magnitude(float(v))


def e2m1_value(code: int) -> float:
    return _load().adahop_ref_e2m1_value(int(code))


def mx_block(y: np.ndarray):
    """(codes[16] uint8, scale byte) of one 32-element fp32 block."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    assert y.shape == (32,)
    codes = np.zeros(16, dtype=np.uint8)
    scale = np.zeros(1, dtype=np.uint8)
    _load().adahop_ref_mx_block(_ptr(y), _ptr(codes), _ptr(scale))
    return codes, int(scale[0])


def iht_quant(src: np.ndarray, contract: int, hadamard_block: int = 32,
              zero_idx=None, zero_axis: int = ROWS):
    """(codes [outer][K/2], scales [outer][K/32], gathered or None)."""
    assert src.dtype == np.uint16 and src.ndim == 2
    src = np.ascontiguousarray(src)
    rows, cols = src.shape
    K, outer = (cols, rows) if contract == COLS else (rows, cols)
    z = np.ascontiguousarray(np.asarray([] if zero_idx is None else zero_idx, dtype=np.int32))
    codes = np.zeros((outer, K // 2), dtype=np.uint8)
    scales = np.zeros((outer, K // 32), dtype=np.uint8)
    gathered = None
    if z.size:
        gathered = np.zeros((z.size, cols) if zero_axis == ROWS else (z.size, rows),
                            dtype=np.uint16)
    _check(_load().adahop_ref_iht_quant(_ptr(src), rows, cols, cols, contract, hadamard_block,
                                        _ptr(z) if z.size else None, z.size, zero_axis,
                                        _ptr(codes), _ptr(scales), _ptr(gathered)),
           "iht_quant")
    return codes, scales, gathered


def _idx64(v, n):
    v = np.arange(n, dtype=np.int64) if v is None else np.ascontiguousarray(v, dtype=np.int64)
    return v


def gemm_mx(a_codes, a_scales, b_codes, b_scales, rows=None, cols=None):
    """fp64 product of packed operands on outputs rows x cols: (C, sum|ab|)."""
    K = a_codes.shape[1] * 2
    assert b_codes.shape[1] * 2 == K
    rows = _idx64(rows, a_codes.shape[0])
    cols = _idx64(cols, b_codes.shape[0])
    C = np.zeros((rows.size, cols.size), dtype=np.float64)
    A = np.zeros_like(C)
    args = [np.ascontiguousarray(x) for x in (a_codes, a_scales, b_codes, b_scales)]
    _check(_load().adahop_ref_gemm_mx(*[_ptr(x) for x in args], K, _ptr(rows), rows.size,
                                      _ptr(cols), cols.size, _ptr(C), _ptr(A)), "gemm_mx")
    return C, A


def gemm_bf16(a, a_trans, b, b_trans, K, rows, cols):
    """fp64 product of bf16 operands: A(i,t) = a[i,t] (a[t,i] if a_trans),
    B(t,j) = b[t,j] (b[j,t] if b_trans); outputs rows x cols."""
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    C = np.zeros((rows.size, cols.size), dtype=np.float64)
    A = np.zeros_like(C)
    _check(_load().adahop_ref_gemm_bf16(_ptr(a), a.shape[1], int(a_trans), _ptr(b), b.shape[1],
                                        int(b_trans), K, _ptr(rows), rows.size, _ptr(cols),
                                        cols.size, _ptr(C), _ptr(A)), "gemm_bf16")
    return C, A


def walk_mx(a_codes, a_scales, b_codes, b_scales, step, rows=None, cols=None):
    """Running-error terms (walk, rmax) of an fp32 accumulation of the packed
    product, `step` products at a time in contraction order (a tolerance for
    the tests; see adahop_ref.h)."""
    K = a_codes.shape[1] * 2
    rows = _idx64(rows, a_codes.shape[0])
    cols = _idx64(cols, b_codes.shape[0])
    W = np.zeros((rows.size, cols.size), dtype=np.float64)
    R = np.zeros_like(W)
    args = [np.ascontiguousarray(x) for x in (a_codes, a_scales, b_codes, b_scales)]
    _check(_load().adahop_ref_walk_mx(*[_ptr(x) for x in args], K, step, _ptr(rows), rows.size,
                                      _ptr(cols), cols.size, _ptr(W), _ptr(R)), "walk_mx")
    return W, R


def walk_bf16(a, a_trans, b, b_trans, K, step, rows, cols):
    """As walk_mx, for the bf16 product of gemm_bf16."""
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    W = np.zeros((rows.size, cols.size), dtype=np.float64)
    R = np.zeros_like(W)
    _check(_load().adahop_ref_walk_bf16(_ptr(a), a.shape[1], int(a_trans), _ptr(b), b.shape[1],
                                        int(b_trans), K, step, _ptr(rows), rows.size, _ptr(cols),
                                        cols.size, _ptr(W), _ptr(R)), "walk_bf16")
    return W, R


def dequant(codes, scales) -> np.ndarray:
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    outer, K = codes.shape[0], codes.shape[1] * 2
    out = np.zeros((outer, K), dtype=np.float64)
    _check(_load().adahop_ref_dequant(_ptr(codes), _ptr(scales), outer, K, _ptr(out)),
           "dequant")
    return out


def bf16_to_f64(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
