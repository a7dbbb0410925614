"""Pins of the oracle's products: the MXFP4 residual product against exact
integer and rational arithmetic, the bf16 product against a library matmul,
and the outlier split (extracted lines + residual = full product) exactly."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import pipeline
from conftest import read_golden


GRID = {int(c, 16): float(v) for c, v in (ln.split() for ln in read_golden("e2m1_grid.txt"))}


def decode(codes, scales):
    """Independent decode from the OCP grid fixture (not the oracle's)."""
    outer, K = codes.shape[0], codes.shape[1] * 2
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(outer, K)
    vals = np.vectorize(GRID.get)(nib)
    return vals * np.ldexp(1.0, np.repeat(scales.astype(np.int64) - 127, 32, axis=1))


def rand_packed(rng, outer, K, scale_lo=120, scale_hi=134):
    codes = rng.integers(0, 256, size=(outer, K // 2), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi, size=(outer, K // 32), dtype=np.uint8)
    return codes, scales


def test_integer_special_case():
    """Scales 2^0 and integer grid values only: an integer matmul, exactly."""
    rng = np.random.default_rng(0)
    ints = [c for c, v in GRID.items() if float(v).is_integer()]
    m, n, K = 13, 9, 96
    a = rng.choice(ints, size=(m, K)); b = rng.choice(ints, size=(n, K))
    pack = lambda x: (x[:, 0::2] | (x[:, 1::2] << 4)).astype(np.uint8)
    ones = lambda r: np.full((r, K // 32), 127, dtype=np.uint8)
    C, absC = oracle.gemm_mx(pack(a), ones(m), pack(b), ones(n))
    va = np.vectorize(GRID.get)(a).astype(np.int64); vb = np.vectorize(GRID.get)(b).astype(np.int64)
    assert np.array_equal(C, (va @ vb.T).astype(np.float64))
    assert np.array_equal(absC, (np.abs(va) @ np.abs(vb).T).astype(np.float64))


def test_rational_exact_small():
    rng = np.random.default_rng(1)
    m, n, K = 5, 4, 64
    ac, as_ = rand_packed(rng, m, K, 100, 150)
    bc, bs = rand_packed(rng, n, K, 100, 150)
    C, _ = oracle.gemm_mx(ac, as_, bc, bs)
    A, B = decode(ac, as_), decode(bc, bs)
    for i in range(m):
        for j in range(n):
            exact = sum(Fraction(A[i, t]) * Fraction(B[j, t]) for t in range(K))
            assert C[i, j] == float(exact)


def test_matches_library_matmul_and_selection():
    rng = np.random.default_rng(2)
    m, n, K = 70, 50, 256
    ac, as_ = rand_packed(rng, m, K)
    bc, bs = rand_packed(rng, n, K)
    ref = decode(ac, as_) @ decode(bc, bs).T
    rows = np.array([0, 5, 69, 33]); cols = np.array([49, 0, 7])
    C, _ = oracle.gemm_mx(ac, as_, bc, bs, rows, cols)
    assert np.allclose(C, ref[np.ix_(rows, cols)], rtol=1e-14, atol=1e-300)
    Cf, _ = oracle.gemm_mx(ac, as_, bc, bs)
    assert np.allclose(Cf, ref, rtol=1e-13, atol=1e-12 * np.abs(ref).max())


def bf(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("a_trans,b_trans", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_bf16_product_layouts(a_trans, b_trans):
    rng = np.random.default_rng(3)
    m, n, K = 11, 7, 40
    A = bf(rng.standard_normal((m, K))); B = bf(rng.standard_normal((K, n)))
    a = A.T.copy() if a_trans else A
    b = B.T.copy() if b_trans else B
    C, _ = oracle.gemm_bf16(a, a_trans, b, b_trans, K, np.arange(m), np.arange(n))
    ref = oracle.bf16_to_f64(A) @ oracle.bf16_to_f64(B)
    assert np.allclose(C, ref, rtol=1e-13, atol=1e-13)


def int_bf16(rng, shape, lo=-6, hi=7):
    return bf(rng.integers(lo, hi, size=shape).astype(np.float32))


def exact_product(op, lhs, rhs):
    L, R = oracle.bf16_to_f64(lhs), oracle.bf16_to_f64(rhs)
    return {"FWD": lambda: L @ R.T, "DGRAD": lambda: L @ R, "WGRAD": lambda: L.T @ R}[op]()


@pytest.mark.parametrize("op,pat_lhs,pat_rhs,route", [
    ("FWD", "R", "N", "OE_LEFT"), ("FWD", "N", "R", "OE_RIGHT"), ("FWD", "C", "N", "OE_INNER"),
    ("DGRAD", "R", "N", "OE_LEFT"), ("DGRAD", "N", "C", "OE_RIGHT"), ("DGRAD", "C", "N", "OE_INNER"),
    ("WGRAD", "C", "N", "OE_LEFT"), ("WGRAD", "R", "C", "OE_RIGHT"), ("WGRAD", "R", "N", "OE_INNER"),
])
def test_outlier_split_identity(op, pat_lhs, pat_rhs, route):
    """On every extracted line the result is the exact bf16 product of the
    original operands (the residual contributes exactly zero there); for
    inner extraction, result - residual product = the exact rank-k term."""
    rng = np.random.default_rng(hash((op, route)) % 2**32)
    T, Din, Dout = 96, 64, 128
    shapes = {"FWD": ((T, Din), (Dout, Din)), "DGRAD": ((T, Dout), (Dout, Din)),
              "WGRAD": ((T, Dout), (T, Din))}[op]
    lhs = int_bf16(rng, shapes[0]); rhs = int_bf16(rng, shapes[1])
    k = 8
    r = pipeline.gemm(op, lhs, rhs, T, Din, Dout, pat_lhs, pat_rhs, route=route, k=k)
    assert r["route"] == route
    idx = r["idx"]
    assert idx.size == k and np.all(np.diff(idx) > 0)
    exact = exact_product(op, lhs, rhs)
    C = r["C"]
    res, _ = oracle.gemm_mx(r["a_codes"], r["a_scales"], r["b_codes"], r["b_scales"])
    if route == "OE_LEFT":
        assert np.all(res[idx, :] == 0)
        assert np.array_equal(C[idx, :], exact[idx, :])
        rest = np.setdiff1d(np.arange(r["m"]), idx)
        assert np.array_equal(C[rest], res[rest])
    elif route == "OE_RIGHT":
        assert np.all(res[:, idx] == 0)
        assert np.array_equal(C[:, idx], exact[:, idx])
        rest = np.setdiff1d(np.arange(r["n"]), idx)
        assert np.array_equal(C[:, rest], res[:, rest])
    else:
        # Inner: A[:, idx] B[idx, :] exactly, from the original values.
        L, R = oracle.bf16_to_f64(lhs), oracle.bf16_to_f64(rhs)
        Ai = {"FWD": L, "DGRAD": L, "WGRAD": L.T}[op][:, idx]
        Bi = {"FWD": R.T, "DGRAD": R, "WGRAD": R}[op][idx, :]
        assert np.array_equal(C - res, Ai @ Bi)
    # The gathered lines are the source bits, one line per row: [k][len].
    tensor, axis = oracle.scan_target(op, route)
    g = r["a_gathered"] if tensor == 0 else r["b_gathered"]
    src = lhs if tensor == 0 else rhs
    assert np.array_equal(g, src[idx, :] if axis == oracle.ROWS else src[:, idx].T)


def test_split_identity_unquantized():
    """The bookkeeping itself: A = A_res + (extracted lines put back), for
    rows and columns, on random bf16 data (fp64, exact)."""
    rng = np.random.default_rng(4)
    t = bf(rng.standard_normal((64, 96)))
    idx = np.array([3, 10, 40], dtype=np.int32)
    for axis in (oracle.ROWS, oracle.COLS):
        # hadamard 0, contraction along the other axis: residual lines are zero codes.
        contract = oracle.COLS if axis == oracle.ROWS else oracle.ROWS
        codes, scales, g = oracle.iht_quant(t, contract, 0, idx, axis)
        deq = oracle.dequant(codes, scales)      # [outer][K]
        if axis == oracle.ROWS:
            assert np.all(deq[idx, :] == 0)
            assert np.array_equal(g, t[idx, :])
        else:
            assert np.all(deq[idx, :] == 0)      # outer = columns here
            assert np.array_equal(g, t[:, idx].T)   # one extracted line per row
    # Zeroing inner lines equals quantizing a copy with those entries zeroed.
    z = t.copy(); z[:, idx] = 0
    c1, s1, _ = oracle.iht_quant(t, oracle.COLS, 32, idx, oracle.COLS)
    c2, s2, _ = oracle.iht_quant(z, oracle.COLS, 32)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_bf16_route_is_exact_product():
    rng = np.random.default_rng(5)
    lhs = bf(rng.standard_normal((64, 32))); rhs = bf(rng.standard_normal((48, 32)))
    r = pipeline.gemm("FWD", lhs, rhs, 64, 32, 48, "R", "R")
    assert r["route"] == "BF16"
    assert np.allclose(r["C"], exact_product("FWD", lhs, rhs), rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("op", ["FWD", "DGRAD", "WGRAD"])
def test_pipeline_close_to_exact(op):
    """A quantized product stays within MXFP4 noise of the exact one, and the
    packed operands follow each op's contraction direction."""
    rng = np.random.default_rng(6)
    T, Din, Dout = 128, 96, 64
    shapes = {"FWD": ((T, Din), (Dout, Din)), "DGRAD": ((T, Dout), (Dout, Din)),
              "WGRAD": ((T, Dout), (T, Din))}[op]
    lhs = bf(rng.standard_normal(shapes[0])); rhs = bf(rng.standard_normal(shapes[1]))
    r = pipeline.gemm(op, lhs, rhs, T, Din, Dout, "N", "N")
    ex = exact_product(op, lhs, rhs)
    assert r["route"] == "IHT"
    assert r["a_codes"].shape == (r["m"], r["K"] // 2) and r["b_codes"].shape == (r["n"], r["K"] // 2)
    err = np.linalg.norm(r["C"] - ex) / np.linalg.norm(ex)
    assert 0.02 < err < 0.3


# ---------------------------------------------------------------------------
# Running-error terms (the tolerance of the GPU comparisons)
# ---------------------------------------------------------------------------
def _walk_direct(prod, step):
    """Straight from the definition, in Python floats: S_j, R_j, walk, rmax."""
    s, r, w = 0.0, 0.0, 0.0
    for t0 in range(0, len(prod), step):
        s += float(sum(prod[t0:t0 + step]))
        r = max(r, abs(s))
        w += abs(s) + r
    return w, r


def test_walk_closed_form():
    # Every product equal to 1 (E2M1 code 0x2 = 1.0, unit scales): S_j = j*step,
    # R_j = S_j, so walk = 2 * step * n(n+1)/2 with n = K/step, and rmax = K.
    K, step = 256, 32
    codes = np.full((3, K // 2), 0x22, dtype=np.uint8)
    scales = np.full((3, K // 32), 127, dtype=np.uint8)
    W, R = oracle.walk_mx(codes, scales, codes, scales, step)
    n = K // step
    assert np.all(W == step * n * (n + 1)) and np.all(R == K)
    # Alternating blocks of +1 and -1 (code 0xA = -1.0 in the high and low
    # nibbles): S_j alternates 32, 0, 32, 0, ...; R_j = 32; walk = sum of
    # |S_j| + 32 = 32 * (n/2) + 32 n.
    b = codes.copy()
    b[:, 16:32] = 0xAA
    b[:, 48:64] = 0xAA
    b[:, 80:96] = 0xAA
    b[:, 112:128] = 0xAA
    W, R = oracle.walk_mx(codes, scales, b, scales, 32)
    assert np.all(W == 32 * 4 + 32 * 8) and np.all(R == 32)


def test_walk_bf16_matches_definition():
    rng = np.random.default_rng(11)
    m, n, K = 6, 5, 100                      # K not a multiple of the step: a short last group
    a = rng.standard_normal((m, K)).astype(np.float32)
    b = rng.standard_normal((K, n)).astype(np.float32)
    from parity import f32_to_bf16_rne, bf16_to_f32
    a16, b16 = f32_to_bf16_rne(a), f32_to_bf16_rne(b)
    W, R = oracle.walk_bf16(a16, 0, b16, 0, K, 8, np.arange(m), np.arange(n))
    av, bv = bf16_to_f32(a16).astype(np.float64), bf16_to_f32(b16).astype(np.float64)
    for i in range(m):
        for j in range(n):
            w, r = _walk_direct(av[i] * bv[:, j], 8)
            assert W[i, j] == pytest.approx(w, rel=1e-12) and R[i, j] == pytest.approx(r, rel=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_walk_bounds_simulated_fp32_accumulators(seed):
    # fp32 accumulators of the shapes the GPU kernels use, simulated with
    # numpy float32: groups of `step` products summed with several fp32
    # roundings inside a group, added in contraction order, the contraction
    # cut into 1-4 contiguous parts added at the end. Every result must lie
    # within u (walk + C_INT sum|ab| + 72 rmax) of the exact sum -- and that
    # bound must be far tighter than the plain (K/step) u sum|ab|.
    from parity import C_INT, U
    rng = np.random.default_rng(100 + seed)
    K, step = 8192, 32
    worst, ratio = 0.0, []
    for trial in range(60):
        x = rng.standard_normal(K) * rng.standard_normal(K)
        if trial % 3 == 0:
            x -= x.mean()                            # cancellation
        if trial % 5 == 0:
            x[rng.integers(0, K, 8)] *= 1e4          # a few huge products
        exact = float(np.sum(x.astype(np.float64)))
        parts = int(rng.integers(1, 5))
        cuts = [0] + sorted(rng.choice(np.arange(step, K, step), parts - 1, replace=False).tolist()) + [K]
        total = np.float32(0.0)
        for p in range(parts):
            acc = np.float32(0.0)
            for t0 in range(cuts[p], cuts[p + 1], step):
                g = x[t0:t0 + step].astype(np.float32)
                inner = np.float32(0.0)
                for v in g:                          # worst case: every product rounded in
                    inner = np.float32(inner + v)
                acc = np.float32(acc + inner)
            total = np.float32(total + acc)
        w, r = _walk_direct(x, step)
        bound = U * (w + C_INT * float(np.sum(np.abs(x))) + 72 * r)
        # roundings inside a group are bounded by step * u * sum|x| over it in
        # this worst-case simulation; the kernels round at most C_INT times
        inner_extra = (step - C_INT) * U * float(np.sum(np.abs(x)))
        err = abs(float(total) - exact)
        assert err <= bound + inner_extra, (trial, err, bound)
        worst = max(worst, err / (bound + inner_extra))
        ratio.append(w / ((K / step) * float(np.sum(np.abs(x)))))
    assert worst < 1.0
    assert np.median(ratio) < 0.2


def test_walk_bounds_one_rounding_per_group():
    # The model the GEMM bar uses: each group's products summed exactly, one
    # fp32 rounding per group addition, parts added afterwards. Here the bound
    # without the inner-group allowance must hold on its own.
    from parity import C_INT, U
    rng = np.random.default_rng(7)
    K, step = 32768, 32
    for trial in range(40):
        x = rng.standard_normal(K) * rng.standard_normal(K)
        if trial % 2:
            x -= x.mean()
        groups = x.reshape(-1, step).sum(axis=1)          # exact enough in fp64
        parts = int(rng.integers(1, 5))
        cuts = np.linspace(0, groups.size, parts + 1).astype(int)
        total = np.float32(0.0)
        for p in range(parts):
            acc = np.float32(0.0)
            for gsum in groups[cuts[p]:cuts[p + 1]]:
                acc = np.float32(acc + np.float32(gsum))
            total = np.float32(total + acc)
        w, r = _walk_direct(x, step)
        bound = U * (w + C_INT * float(np.sum(np.abs(x))) + 72 * r)
        assert abs(float(total) - float(np.sum(x))) <= bound
