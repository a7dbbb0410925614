"""One AdaHOP GEMM call, composed from the oracle's steps.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Follows the four-stage pipeline of "AdaHOP: Fast and Accurate Low-Precision
Training via Outlier-Pattern-Aware Rotation" (arXiv 2604.02525), Fig. 9 and
the appendix list of its kernels: FOID picks the outlier lines; the residual
(those lines zeroed) is rotated by the 32-point IHT along the inner dimension
and quantized to MXFP4; the residual product runs on the dequantized operands;
the outlier product runs in high precision on the extracted bf16 lines and is
scatter-added into the result. Fig. 5 fixes which product each pattern pair
gets.

Frames. A linear layer Y = X W^T has three products (Table 1's columns):
  FWD   C = Y  [T, Dout]  = A B with A = X [T,Din],     B = W^T,  K = Din
  DGRAD C = dX [T, Din]   = A B with A = GY [T,Dout],   B = W,    K = Dout
  WGRAD C = dW [Dout,Din] = A B with A = GY^T,          B = X,    K = T
Packed operands are K-contiguous: A as [m][K], B as [n][K].
"""
import numpy as np

from . import (COLS, ROWS, dequant, foid, gemm_bf16, gemm_mx, iht_quant, route as
               route_of, scan_target, walk_bf16, walk_mx)

# Granularity of the running-error terms that bound an fp32 accumulator (a
# tolerance for comparisons, not part of the method): the FP4 product is
# accumulated at most one 32-element MX block at a time (each block's products
# share one scale and sum exactly), the bf16 products 8 at a time at most.
FP4_STEP = 32
BF16_STEP = 8

# Per op: (m, n, K) from (T, Din, Dout); the axis of each stored tensor that the
# contraction runs along; and whether the textbook operand is the stored tensor
# transposed.
_SHAPES = {
    "FWD": lambda T, Din, Dout: (T, Dout, Din),
    "DGRAD": lambda T, Din, Dout: (T, Din, Dout),
    "WGRAD": lambda T, Din, Dout: (Dout, Din, T),
}
_CONTRACT = {"FWD": (COLS, COLS), "DGRAD": (COLS, ROWS), "WGRAD": (ROWS, ROWS)}
# A(i,t) = lhs[i,t] unless a_trans; B(t,j) = rhs[t,j] unless b_trans.
_TRANS = {"FWD": (0, 1), "DGRAD": (0, 0), "WGRAD": (1, 0)}


def gemm(op, lhs, rhs, T, Din, Dout, pat_lhs="N", pat_rhs="N", route=None, k=64,
         rows=None, cols=None, probe=64):
    """Reference result of one call on outputs rows x cols (all if None).

    Returns a dict with the route, the FOID indices, the packed operands A and
    B (codes, scales), the gathered bf16 lines, C (fp64), and per output the
    terms of the fp32 accumulation-error bound: absC (the sum of |products|),
    walk and rmax (running-error terms, FP4_STEP / BF16_STEP at a time) and
    k_inner (the rank of an inner outlier term added after the residual).
    """
    lhs = np.ascontiguousarray(lhs)
    rhs = np.ascontiguousarray(rhs)
    m, n, K = _SHAPES[op](T, Din, Dout)
    r = route or route_of(op, pat_lhs, pat_rhs)
    rows = np.arange(m, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(n, dtype=np.int64) if cols is None else np.asarray(cols, dtype=np.int64)
    a_trans, b_trans = _TRANS[op]
    out = {"route": r, "m": m, "n": n, "K": K, "idx": None,
           "a_gathered": None, "b_gathered": None}

    out["k_inner"] = 0
    if r == "BF16":
        # Both operands hurt: the plain high-precision product (Fig. 5).
        C, absC = gemm_bf16(lhs, a_trans, rhs, b_trans, K, rows, cols)
        walk, rmax = walk_bf16(lhs, a_trans, rhs, b_trans, K, BF16_STEP, rows, cols)
        out.update(C=C, absC=absC, walk=walk, rmax=rmax)
        return out

    # Stage 1, FOID: which stored tensor and axis hold the extracted lines.
    zero = {0: None, 1: None}           # tensor -> (idx, axis)
    if r in ("OE_LEFT", "OE_RIGHT", "OE_INNER"):
        tensor, axis = scan_target(op, r)
        idx = foid(lhs if tensor == 0 else rhs, axis, k, probe)
        out["idx"] = idx
        zero[tensor] = (idx, axis)
        if r == "OE_INNER":
            # The matching inner lines of the other operand leave the residual too.
            # Inner lines of the rhs are indexed along its contraction axis.
            zero[1] = (idx, _CONTRACT[op][1])

    # Stage 2, IHT + MXFP4 quantization of both residuals.
    had = 0 if r == "MXFP4" else 32
    packed = []
    for t, src in ((0, lhs), (1, rhs)):
        z = zero[t]
        codes, scales, gathered = iht_quant(src, _CONTRACT[op][t], had,
                                            None if z is None else z[0],
                                            ROWS if z is None else z[1])
        packed.append((codes, scales))
        out["a_gathered" if t == 0 else "b_gathered"] = gathered
    (ac, as_), (bc, bs) = packed
    out.update(a_codes=ac, a_scales=as_, b_codes=bc, b_scales=bs)

    # Stage 3, the residual product on the dequantized operands.
    C, absC = gemm_mx(ac, as_, bc, bs, rows, cols)
    walk, rmax = walk_mx(ac, as_, bc, bs, FP4_STEP, rows, cols)

    # Stage 3 (outlier half) + stage 4: the bf16 outlier product, scatter-added.
    idx = out["idx"]
    if r == "OE_LEFT":
        # Rows idx of A, gathered one line per row: A_g(p,t) = g[p][t].
        g = out["a_gathered"]
        hit = np.nonzero(np.isin(rows, idx))[0]
        if hit.size:
            pos = np.searchsorted(idx, rows[hit])
            oe, oabs = gemm_bf16(g, 0, rhs, b_trans, K, pos, cols)
            C[hit, :] += oe
            absC[hit, :] += oabs
            w, rm = walk_bf16(g, 0, rhs, b_trans, K, BF16_STEP, pos, cols)
            walk[hit, :] += w
            rmax[hit, :] += rm
    elif r == "OE_RIGHT":
        # Columns idx of B, one line per row: B_g(t,p) = g[p][t].
        g = out["b_gathered"]
        hit = np.nonzero(np.isin(cols, idx))[0]
        if hit.size:
            pos = np.searchsorted(idx, cols[hit])
            oe, oabs = gemm_bf16(lhs, a_trans, g, 1, K, rows, pos)
            C[:, hit] += oe
            absC[:, hit] += oabs
            w, rm = walk_bf16(lhs, a_trans, g, 1, K, BF16_STEP, rows, pos)
            walk[:, hit] += w
            rmax[:, hit] += rm
    elif r == "OE_INNER":
        ga, gb = out["a_gathered"], out["b_gathered"]
        kk = idx.size
        # Inner lines, one per row: A_g(i,p) = ga[p][i], B_g(p,j) = gb[p][j].
        oe, oabs = gemm_bf16(ga, 1, gb, 0, kk, rows, cols)
        C += oe
        absC += oabs
        w, rm = walk_bf16(ga, 1, gb, 0, kk, BF16_STEP, rows, cols)
        walk += w
        rmax += rm
        out["k_inner"] = kk
    out.update(C=C, absC=absC, walk=walk, rmax=rmax)
    return out


def dequantized_product(a_codes, a_scales, b_codes, b_scales) -> np.ndarray:
    """Full fp64 product deq(A) deq(B)^T via a library matmul (small sizes)."""
    return dequant(a_codes, a_scales) @ dequant(b_codes, b_scales).T


# ---------------------------------------------------------------------------
# Saved forward context (appendix item on IHT and quantization: for the
# activation of the forward path, the quantized residual and the bf16 outlier
# tensor are kept for backpropagation).
#
# Reading: the backward's only product that reads the activation X [T, Din]
# is the weight gradient dW = GY^T X, which contracts over T. What is kept is
# therefore X in the form that product consumes: FOID's extracted columns
# (when the weight gradient's route extracts X's columns, OE-Right), the
# residual with those columns zeroed, rotated and MXFP4-quantized along T, and
# the extracted columns in bf16. Routes that would need X in bf16 in the
# backward (BF16; OE-Left, whose outlier product multiplies GY's lines by the
# whole of X; OE-Inner, which cuts X's rows) keep no context.
# ---------------------------------------------------------------------------
CONTEXT_ROUTES = ("IHT", "MXFP4", "OE_RIGHT")


def forward_context(X, pat_gy="N", pat_x="N", route=None, k=64, probe=64):
    """The context kept for the weight gradient of X [T, Din]: dict with the
    weight gradient's route, idx (or None), codes [Din][T/2], scales
    [Din][T/32] (blocks along T, one row per column of X) and lines [k][T]
    (X's extracted columns, bf16) or None."""
    X = np.ascontiguousarray(X)
    r = route or route_of("WGRAD", pat_gy, pat_x)
    if r not in CONTEXT_ROUTES:
        raise ValueError(f"no context for a weight gradient on route {r}")
    idx = None
    if r == "OE_RIGHT":
        tensor, axis = scan_target("WGRAD", r)
        assert tensor == 1 and axis == COLS      # X's columns
        idx = foid(X, COLS, k, probe)
    had = 0 if r == "MXFP4" else 32
    codes, scales, lines = iht_quant(X, ROWS, had, idx, COLS)
    return {"route": r, "idx": idx, "codes": codes, "scales": scales, "lines": lines}


def context_bytes(T, Din, k, route):
    """Bytes of the context's arrays (without alignment): indices, codes,
    scales and lines."""
    ext = route == "OE_RIGHT"
    return (4 * k if ext else 0) + Din * T // 2 + Din * T // 32 + (2 * k * T if ext else 0)


def wgrad_from_context(GY, ctx, T, Din, Dout, pat_gy="N", rows=None, cols=None):
    """dW = GY^T X with X taken from its saved context: the weight gradient's
    remaining steps (GY's quantization along T, the residual product, the
    outlier product GY^T X[:, idx] on the kept lines, the scatter-add), as in
    gemm() for the same route."""
    GY = np.ascontiguousarray(GY)
    r = ctx["route"]
    m, n, K = Dout, Din, T
    rows = np.arange(m, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(n, dtype=np.int64) if cols is None else np.asarray(cols, dtype=np.int64)
    had = 0 if r == "MXFP4" else 32
    ac, as_, _ = iht_quant(GY, ROWS, had)
    C, absC = gemm_mx(ac, as_, ctx["codes"], ctx["scales"], rows, cols)
    walk, rmax = walk_mx(ac, as_, ctx["codes"], ctx["scales"], FP4_STEP, rows, cols)
    if r == "OE_RIGHT":
        idx, g = ctx["idx"], ctx["lines"]
        hit = np.nonzero(np.isin(cols, idx))[0]
        if hit.size:
            pos = np.searchsorted(idx, cols[hit])
            oe, oabs = gemm_bf16(GY, 1, g, 1, K, rows, pos)
            C[:, hit] += oe
            absC[:, hit] += oabs
            w, rm = walk_bf16(GY, 1, g, 1, K, BF16_STEP, rows, pos)
            walk[:, hit] += w
            rmax[:, hit] += rm
    return {"route": r, "m": m, "n": n, "K": K, "a_codes": ac, "a_scales": as_, "C": C,
            "absC": absC, "walk": walk, "rmax": rmax, "k_inner": 0}
