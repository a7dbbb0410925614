"""Pins of the saved forward context (appendix item on IHT and quantization:
the forward keeps the activation's quantized residual and its bf16 outlier
tensor for backpropagation), in the oracle's reading: X [T, Din] kept as
the weight gradient consumes it, rotated and MXFP4-quantized along T with the
extracted columns zeroed, plus those columns in bf16.

Pinned against what the format and the mathematics fix, not against the
oracle itself: the extracted columns are X's own bits; the kept residual
reconstructs X within the MXFP4 rounding bound of each block (E2M1 with the
OCP scale rule: per element at most 2^(s+1) after scaling, orthonormal
rotation preserves the block's L2 error); the memory is 17/32 bytes per
element plus the lines; the weight gradient from the context equals the
weight gradient from X."""
import numpy as np
import pytest

import oracle
import synth
from oracle import pipeline


def make_x(T, Din, seed, n_cols=3):
    lines = synth.pick_lines(seed, 31, Din, n_cols)
    return synth.fill_bf16(T, Din, seed, 30, 1.0, 1, lines, 50.0), np.sort(lines)


def make_gy(T, Dout, seed):
    lines = synth.pick_lines(seed, 33, T, max(1, T // 200))
    return synth.fill_bf16(T, Dout, seed, 32, 1e-3, 0, lines, 100.0)


def inverse_rotation(y):
    """Orthonormal Sylvester H_32 / sqrt(32) along the last axis (fp64; the
    matrix is symmetric and its own inverse)."""
    H = np.array([[(-1) ** bin(i & j).count("1") for j in range(32)] for i in range(32)], dtype=np.float64)
    return (y.reshape(*y.shape[:-1], -1, 32) @ (H / np.sqrt(32))).reshape(y.shape)


@pytest.mark.parametrize("route", ["OE_RIGHT", "IHT", "MXFP4"])
def test_context_reconstructs_x(route):
    T, Din, k = 256, 96, 4
    X, planted = make_x(T, Din, 3)
    ctx = pipeline.forward_context(X, "R", "C", route, k)
    xd = oracle.bf16_to_f64(X)
    deq = oracle.dequant(ctx["codes"], ctx["scales"])          # [Din][T], rotated along T
    rec = inverse_rotation(deq) if route != "MXFP4" else deq
    res = xd.T.copy()                                            # residual, one row per column of X
    if route == "OE_RIGHT":
        idx = ctx["idx"]
        assert idx.size == k and np.all(np.diff(idx) > 0)
        assert set(planted) <= set(idx.tolist())                 # the planted columns are extracted
        assert np.array_equal(ctx["lines"], np.ascontiguousarray(X[:, idx].T))   # bit for bit
        res[idx, :] = 0.0
        assert np.all(ctx["codes"][idx] == 0) and np.all(ctx["scales"][idx] == 0)
    else:
        assert ctx["idx"] is None and ctx["lines"] is None
    # per 32-block of a column: L2 error <= sqrt(32) * 2^(s+1) (+ fp32 rotation slack)
    s = ctx["scales"].astype(np.int64) - 127                     # [Din][T/32]
    err = (rec - res).reshape(Din, T // 32, 32)
    bound = np.sqrt(32) * np.ldexp(1.0, s + 1) * (1 + 1e-6) + 1e-6 * np.abs(res).reshape(Din, T // 32, 32).sum(-1)
    nz = ctx["scales"] > 0
    assert np.all(np.linalg.norm(err, axis=-1)[nz] <= bound[nz])
    assert np.all(err[~nz] == 0)


def test_context_memory():
    for T, Din, k, route in ((32768, 14336, 64, "OE_RIGHT"), (4096, 4096, 64, "OE_RIGHT"),
                             (32768, 4096, 64, "IHT")):
        b = pipeline.context_bytes(T, Din, k, route)
        ext = route == "OE_RIGHT"
        assert b == Din * T * 17 // 32 + (4 * k + 2 * k * T if ext else 0)
        assert 3.5 < 2 * T * Din / b <= 64 / 17                  # against bf16 X: at most 3.76x


@pytest.mark.parametrize("route", ["OE_RIGHT", "IHT", "MXFP4"])
def test_wgrad_from_context_equals_wgrad(route):
    T, Din, Dout, k = 256, 96, 64, 4
    X, _ = make_x(T, Din, 5)
    GY = make_gy(T, Dout, 5)
    ctx = pipeline.forward_context(X, "R", "C", route, k)
    a = pipeline.wgrad_from_context(GY, ctx, T, Din, Dout, "R")
    b = pipeline.gemm("WGRAD", GY, X, T, Din, Dout, "R", "C", route=route, k=k)
    assert a["route"] == b["route"] == route
    for key in ("a_codes", "a_scales"):
        assert np.array_equal(a[key], b[key])
    assert np.array_equal(ctx["codes"], b["b_codes"]) and np.array_equal(ctx["scales"], b["b_scales"])
    assert np.array_equal(a["C"], b["C"])


def test_context_refuses_routes_that_need_x_in_bf16():
    X, _ = make_x(64, 32, 1)
    for route in ("BF16", "OE_LEFT", "OE_INNER"):
        with pytest.raises(ValueError):
            pipeline.forward_context(X, "R", "C", route, 4)
    with pytest.raises(ValueError):
        pipeline.forward_context(X, "C", "C")         # CC -> BF16 for the weight gradient
