"""GPU vs oracle parity of each stage and of whole AdaHOP products, on seeded
inputs, at sizes the oracle finishes in seconds (several tiles plus ragged
tails). Bit-exact: FOID indices, MXFP4 codes and scales, gathered lines.
Outputs: the GEMM bar in tests/parity.py."""
import numpy as np
import pytest
import torch

import mxfp4_precision_gemms_amd as A
import oracle
import synth
from oracle import pipeline
from oracle.pipeline import BF16_STEP, FP4_STEP
from parity import bf16_to_f32, check_bf16, check_f32, describe, f32_to_bf16_rne, gamma, gamma_of

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def dev_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def rand_bf16(rng, shape, scale=1.0, planted=None, factor=50.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    if planted is not None:
        axis, lines = planted
        if axis == 0:
            x[lines, :] *= factor
        else:
            x[:, lines] *= factor
    return f32_to_bf16_rne(x)


# --------------------------------------------------------------------------
# IHT + MXFP4 quantization (with zeroing and gathering)
# --------------------------------------------------------------------------
QUANT_CASES = [
    # rows, cols, contract, hadamard, zero_axis, nzero
    (64, 512, "COLS", 32, None, 0),
    (37, 96, "COLS", 32, None, 0),          # ragged rows, K = 96
    (300, 4160, "COLS", 32, "ROWS", 7),     # K spans 3 workgroup chunks, ragged
    (300, 4160, "COLS", 32, "COLS", 9),
    (128, 2048, "COLS", 0, "ROWS", 5),      # no rotation (plain MXFP4)
    (96, 200, "ROWS", 32, None, 0),         # K = 96 down columns, ragged outer
    (544, 130, "ROWS", 32, "COLS", 6),
    (544, 130, "ROWS", 32, "ROWS", 11),
    (1024, 64, "ROWS", 0, "COLS", 3),
    (32, 8, "ROWS", 32, None, 0),           # one block per column
]


@pytest.mark.parametrize("case", QUANT_CASES, ids=[str(c) for c in QUANT_CASES])
def test_iht_quant_bit_exact(case):
    rows, cols, contract, had, zaxis, nz = case
    rng = np.random.default_rng(rows * 7 + cols)
    src = rand_bf16(rng, (rows, cols), planted=(1, rng.choice(cols, 2, replace=False)))
    zidx = None
    if nz:
        dim = rows if zaxis == "ROWS" else cols
        zidx = np.sort(rng.choice(dim, nz, replace=False)).astype(np.int32)
    say("iht_quant", case)
    codes, scales, gathered = A.adahop_iht_quant(
        dev_bf16(src), contract, had,
        None if zidx is None else torch.from_numpy(zidx).to(DEV), zaxis or "ROWS")
    torch.cuda.synchronize()
    rc, rs, rg = oracle.iht_quant(src, oracle.COLS if contract == "COLS" else oracle.ROWS, had,
                                  zidx, oracle.ROWS if zaxis in (None, "ROWS") else oracle.COLS)
    assert np.array_equal(host(codes), rc)
    assert np.array_equal(host(scales), rs)
    if nz:
        assert np.array_equal(host(gathered), rg)


def all_finite_bf16(limit_exp=None):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    keep = exp != 0xFF
    if limit_exp is not None:
        keep &= exp < limit_exp
    return bits[keep]


@pytest.mark.parametrize("had", [0, 32])
@pytest.mark.parametrize("contract", ["COLS", "ROWS"])
def test_iht_quant_every_bf16_pattern(had, contract):
    """Every finite bf16 value (subnormals, signed zeros, extremes) in random
    blocks; with the rotation the magnitudes stay below 2^100 so that no
    butterfly overflows (non-finite inputs are outside the contract)."""
    vals = all_finite_bf16(None if had == 0 else 127 + 100)
    rng = np.random.default_rng(had + len(contract))
    reps = []
    for _ in range(3):
        reps.append(rng.permutation(vals))
    # Also whole blocks of tiny values so that a block scale clamps.
    tiny = vals[((vals >> 7) & 0xFF) < 3]
    reps.append(rng.permutation(np.tile(tiny, 4)))
    flat = np.concatenate(reps)
    flat = flat[: flat.size // 4096 * 4096]
    src = flat.reshape(-1, 256) if contract == "COLS" else flat.reshape(256, -1)
    say("iht_quant every bf16", had, contract, src.shape)
    codes, scales, _ = A.adahop_iht_quant(dev_bf16(src), contract, had)
    torch.cuda.synchronize()
    rc, rs, _ = oracle.iht_quant(src, oracle.COLS if contract == "COLS" else oracle.ROWS, had)
    assert np.array_equal(host(scales), rs)
    assert np.array_equal(host(codes), rc)


# --------------------------------------------------------------------------
# FOID
# --------------------------------------------------------------------------
FOID_CASES = [
    # rows, cols, axis, k, probe, integer-valued (ties)
    (64, 512, "COLS", 16, 64, False),
    (200, 333, "COLS", 40, 64, True),
    (333, 200, "ROWS", 40, 64, True),
    (40, 1000, "COLS", 64, 64, False),       # columns shorter than the probe (P = 40)
    (100, 5000, "COLS", 64, 64, False),      # two selection levels
    (70000, 64, "ROWS", 64, 64, False),      # three levels
    (9000, 128, "ROWS", 1024, 64, True),     # k at its maximum
    (128, 300, "COLS", 300, 64, False),      # k = all candidates
    (96, 256, "ROWS", 7, 16, True),          # shorter probe
    (64, 14336, "COLS", 64, 64, False),      # Llama3.1-8B d_ff columns: 14 chunks, then one
    (1024, 64, "ROWS", 64, 64, True),        # exactly one chunk: scores and selection in one launch
    (64, 4096, "COLS", 64, 64, False),       # 16 chunks of 256 (one candidate per thread), then the final workgroup
    (3000, 64, "ROWS", 32, 64, True),        # chunks of 256 with a ragged last chunk, ties
    (2500, 96, "ROWS", 64, 16, False),       # the same with a short probe (one candidate at a time)
    (64, 8192, "COLS", 64, 64, True),        # 16 chunks of 512, one candidate per thread, ties
    (4097, 64, "ROWS", 64, 64, False),       # 9 chunks of 512, the last holding one candidate
    (64, 4096, "COLS", 128, 64, False),      # k = 128: chunks of 512 (256 < 4 k), 1024 survivors
    (5000, 64, "ROWS", 100, 64, True),       # k = 100: 10 chunks of 512, 1000 survivors, ties
]


@pytest.mark.parametrize("case", FOID_CASES, ids=[str(c) for c in FOID_CASES])
def test_foid_bit_exact(case):
    rows, cols, axis, k, probe, ints = case
    rng = np.random.default_rng(rows + cols + k)
    if ints:
        t = f32_to_bf16_rne(rng.integers(-3, 4, size=(rows, cols)).astype(np.float32))
    else:
        dim = cols if axis == "COLS" else rows
        lines = rng.choice(dim, min(dim, 2 * k), replace=False)
        t = rand_bf16(rng, (rows, cols), planted=(1 if axis == "COLS" else 0, lines),
                      factor=rng.uniform(1, 3))
    say("foid", case)
    idx = A.adahop_detect(dev_bf16(t), axis, k, probe)
    torch.cuda.synchronize()
    ref = oracle.foid(t, oracle.COLS if axis == "COLS" else oracle.ROWS, k, probe)
    assert np.array_equal(host(idx), ref)


@pytest.mark.parametrize("case", [(64, 14336, "COLS"), (70000, 64, "ROWS")],
                         ids=["14-chunks-then-final", "three-levels"])
def test_foid_handoff_fresh_each_call(case):
    # The level before the final one hands its survivors to its last
    # workgroup inside the launch. Back-to-back calls on one workspace, each
    # with other planted lines, must each see their own survivors: a stale
    # read would return an earlier call's indices.
    rows, cols, axis = case
    k = 64
    dim = cols if axis == "COLS" else rows
    ws = torch.empty(max(A.adahop_detect_workspace_size(rows, cols, axis, k), 1), dtype=torch.uint8,
                     device=DEV)
    inputs, outs = [], []
    for it in range(8):
        rng = np.random.default_rng(7000 + it)
        lines = rng.choice(dim, 2 * k, replace=False)
        t = rand_bf16(rng, (rows, cols), planted=(1 if axis == "COLS" else 0, lines),
                      factor=rng.uniform(1, 3))
        inputs.append(t)
    devs = [dev_bf16(t) for t in inputs]
    torch.cuda.synchronize()
    say("foid hand-off", case)
    for d in devs:
        outs.append(A.adahop_detect(d, axis, k, ws=ws).clone())
    torch.cuda.synchronize()
    for t, got in zip(inputs, outs):
        ref = oracle.foid(t, oracle.COLS if axis == "COLS" else oracle.ROWS, k, 64)
        assert np.array_equal(host(got), ref)


# --------------------------------------------------------------------------
# Pre-quantized GEMM with and without the outlier term
# --------------------------------------------------------------------------
def packed_operands(rng, m, n, K):
    a = rand_bf16(rng, (m, K), planted=(1, rng.choice(K, 3, replace=False)))
    b = rand_bf16(rng, (n, K), scale=0.02)
    ac, as_, _ = oracle.iht_quant(a, oracle.COLS, 32)
    bc, bs, _ = oracle.iht_quant(b, oracle.COLS, 32)
    return a, b, ac, as_, bc, bs


# K % 512 == 0 runs the LDS-ring kernel (ragged edges included), other K the
# register-staged kernel (K tails included). With few tiles and K of 4096 or
# more, the ring kernel splits its tiles along K into 2 (300 x 520 x 4096) or
# 4 (520 x 300 x 8192) parts that the fixup kernel adds.
GEMM_CASES = [(256, 128, 128), (512, 384, 512), (300, 200, 96), (33, 1000, 160), (1024, 256, 1024),
              (300, 520, 1024), (77, 1000, 512), (520, 300, 2048), (256, 256, 768),
              (300, 520, 4096), (520, 300, 8192),
              (300, 260, 512), (260, 516, 1024)]   # n % 8 == 4: bf16 rows not 16-byte aligned


@pytest.mark.parametrize("m,n,K", GEMM_CASES)
def test_gemm_mx(m, n, K):
    rng = np.random.default_rng(m + n + K)
    _, _, ac, as_, bc, bs = packed_operands(rng, m, n, K)
    ref, absC = oracle.gemm_mx(ac, as_, bc, bs)
    walk, rmax = oracle.walk_mx(ac, as_, bc, bs, FP4_STEP)
    g = gamma(absC, walk, rmax)
    d = [torch.from_numpy(x).to(DEV) for x in (ac, as_, bc, bs)]
    say("gemm_mx f32", m, n, K)
    c32 = A.adahop_gemm_mx(*d, out_dtype=torch.float32)
    say("gemm_mx bf16", m, n, K)
    c16 = A.adahop_gemm_mx(*d, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    C32, C16 = host(c32), host(c16)
    check_f32(C32, ref, g, "gemm f32")
    say("  " + describe(check_bf16(C16, ref, g, "gemm bf16")))
    # One rounding: the bf16 output is the fp32 result rounded to nearest even.
    assert np.array_equal(C16, f32_to_bf16_rne(C32))


@pytest.mark.parametrize("K", [256, 4096])
@pytest.mark.parametrize("route", ["OE_LEFT", "OE_RIGHT", "OE_INNER"])
def test_gemm_mx_outlier_term(route, K):
    # K = 4096: two K-halves per tile, the outlier term added once by the fixup.
    m, n, k = 320, 192, 12
    rng = np.random.default_rng(5)
    a, b, ac, as_, bc, bs = packed_operands(rng, m, n, K)
    ref, absC = oracle.gemm_mx(ac, as_, bc, bs)
    walk, rmax = oracle.walk_mx(ac, as_, bc, bs, FP4_STEP)
    k_inner = 0
    if route == "OE_LEFT":
        idx = np.sort(rng.choice(m, k, replace=False)).astype(np.int32)
        la = rand_bf16(rng, (k, K))                      # (p, t)
        oe_ref, oe_abs = oracle.gemm_bf16(la, 0, b, 1, K, np.arange(k), np.arange(n))
        w, r = oracle.walk_bf16(la, 0, b, 1, K, BF16_STEP, np.arange(k), np.arange(n))
        ref[idx, :] += oe_ref; absC[idx, :] += oe_abs; walk[idx, :] += w; rmax[idx, :] += r
        oe = {"route": route, "k": k, "idx": torch.from_numpy(idx).to(DEV),
              "a": (dev_bf16(la), True), "b": (dev_bf16(b), True)}
    elif route == "OE_RIGHT":
        idx = np.sort(rng.choice(n, k, replace=False)).astype(np.int32)
        lbT = rand_bf16(rng, (K, k))                     # (t, p) stored t-major
        oe_ref, oe_abs = oracle.gemm_bf16(a, 0, lbT, 0, K, np.arange(m), np.arange(k))
        w, r = oracle.walk_bf16(a, 0, lbT, 0, K, BF16_STEP, np.arange(m), np.arange(k))
        ref[:, idx] += oe_ref; absC[:, idx] += oe_abs; walk[:, idx] += w; rmax[:, idx] += r
        oe = {"route": route, "k": k, "idx": torch.from_numpy(idx).to(DEV),
              "a": (dev_bf16(a), True), "b": (dev_bf16(lbT), False)}
    else:
        ga = rand_bf16(rng, (m, k)); gb = rand_bf16(rng, (n, k))
        oe_ref, oe_abs = oracle.gemm_bf16(ga, 0, gb, 1, k, np.arange(m), np.arange(n))
        w, r = oracle.walk_bf16(ga, 0, gb, 1, k, BF16_STEP, np.arange(m), np.arange(n))
        ref += oe_ref; absC += oe_abs; walk += w; rmax += r; k_inner = k
        oe = {"route": route, "k": k, "a": (dev_bf16(ga), True), "b": (dev_bf16(gb), True)}
    d = [torch.from_numpy(x).to(DEV) for x in (ac, as_, bc, bs)]
    say("gemm_mx outlier", route, K)
    c32 = A.adahop_gemm_mx(*d, oe=oe, out_dtype=torch.float32)
    c16 = A.adahop_gemm_mx(*d, oe=oe, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    g = gamma(absC, walk, rmax, k_inner)
    check_f32(host(c32), ref, g, route)
    say("  " + describe(check_bf16(host(c16), ref, g, route)))
    assert np.array_equal(host(c16), f32_to_bf16_rne(host(c32)))


@pytest.mark.parametrize("K", [512, 4096, 8192])
@pytest.mark.parametrize("route", ["OE_LEFT", "OE_RIGHT"])
def test_gemm_mx_outlier_items_in_kernel(route, K):
    # The outlier product with its wide factor stored across K and its lines
    # along K runs as work items of the GEMM kernel (K % 512 == 0). The packed
    # operands are random, so the extracted lines' residual is not zero: the
    # result must still be residual + outlier product, rounded once. K = 4096
    # and 8192 split the last round's tiles (residual kept by the fixup).
    m, n, k = 320, 520, 12
    rng = np.random.default_rng(9)
    a, b, ac, as_, bc, bs = packed_operands(rng, m, n, K)
    ref, absC = oracle.gemm_mx(ac, as_, bc, bs)
    walk, rmax = oracle.walk_mx(ac, as_, bc, bs, FP4_STEP)
    if route == "OE_LEFT":
        idx = np.sort(rng.choice(m, k, replace=False)).astype(np.int32)
        la = rand_bf16(rng, (k, K))                      # lines (p, t), along K
        bT = np.ascontiguousarray(b.T)                   # B (j, t) stored across K: [K][n]
        oe_ref, oe_abs = oracle.gemm_bf16(la, 0, bT, 0, K, np.arange(k), np.arange(n))
        w, r = oracle.walk_bf16(la, 0, bT, 0, K, BF16_STEP, np.arange(k), np.arange(n))
        ref[idx, :] += oe_ref; absC[idx, :] += oe_abs; walk[idx, :] += w; rmax[idx, :] += r
        oe = {"route": route, "k": k, "idx": torch.from_numpy(idx).to(DEV),
              "a": (dev_bf16(la), True), "b": (dev_bf16(bT), False)}
    else:
        idx = np.sort(rng.choice(n, k, replace=False)).astype(np.int32)
        aT = np.ascontiguousarray(a.T)                   # A (i, t) stored across K: [K][m]
        lb = rand_bf16(rng, (k, K))                      # lines (p, t), along K
        oe_ref, oe_abs = oracle.gemm_bf16(aT, 1, lb, 1, K, np.arange(m), np.arange(k))
        w, r = oracle.walk_bf16(aT, 1, lb, 1, K, BF16_STEP, np.arange(m), np.arange(k))
        ref[:, idx] += oe_ref; absC[:, idx] += oe_abs; walk[:, idx] += w; rmax[:, idx] += r
        oe = {"route": route, "k": k, "idx": torch.from_numpy(idx).to(DEV),
              "a": (dev_bf16(aT), False), "b": (dev_bf16(lb), True)}
    d = [torch.from_numpy(x).to(DEV) for x in (ac, as_, bc, bs)]
    say("gemm_mx outlier items", route, K)
    c32 = A.adahop_gemm_mx(*d, oe=oe, out_dtype=torch.float32)
    c16 = A.adahop_gemm_mx(*d, oe=oe, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    g = gamma(absC, walk, rmax)
    check_f32(host(c32), ref, g, route)
    say("  " + describe(check_bf16(host(c16), ref, g, route)))
    assert np.array_equal(host(c16), f32_to_bf16_rne(host(c32)))


# --------------------------------------------------------------------------
# Whole products: every op x route family, bit-exact intermediates
# --------------------------------------------------------------------------
def operands(op, T, Din, Dout, pl, pr, seed):
    shapes = {"FWD": ((T, Din), (Dout, Din)), "DGRAD": ((T, Dout), (Dout, Din)),
              "WGRAD": ((T, Dout), (T, Din))}[op]
    sig = {"FWD": (1.0, 0.02), "DGRAD": (1e-3, 0.02), "WGRAD": (1e-3, 1.0)}[op]
    out = []
    for t, (pat, shape, s) in enumerate(zip((pl, pr), shapes, sig)):
        axis = {"R": 0, "C": 1, "N": -1}[pat]
        dim = shape[0] if pat == "R" else shape[1]
        lines = synth.pick_lines(seed, 50 + t, dim, max(1, dim // 100)) if pat != "N" else None
        out.append(synth.fill_bf16(shape[0], shape[1], seed, 60 + t, s, axis, lines, 50.0))
    return out


def run_and_compare(op, lhs, rhs, T, Din, Dout, pl, pr, route, k, rows=None, cols=None,
                    oe_in_quant=False):
    say("adahop_gemm", op, (T, Din, Dout), pl + pr, route, k, "oe_in_quant" if oe_in_quant else "")
    plan = A.adahop_gemm_plan(op, T, Din, Dout, pl, pr, route, k, oe_in_quant)
    if oe_in_quant:
        assert plan.oe_in_quant == 1
    if plan.route != A.ROUTE["BF16"]:
        assert plan.layout == (A.LAYOUT_KCHUNK if plan.K % 512 == 0 else A.LAYOUT_ROWS)
    ws = torch.zeros(max(plan.ws_bytes, 1), dtype=torch.uint8, device=DEV)
    L, R = dev_bf16(lhs), dev_bf16(rhs)
    c32 = A.adahop_gemm(op, L, R, pl, pr, route, k, out_dtype=torch.float32, ws=ws,
                        oe_in_quant=oe_in_quant)
    c16 = A.adahop_gemm(op, L, R, pl, pr, route, k, out_dtype=torch.bfloat16,
                        oe_in_quant=oe_in_quant)
    torch.cuda.synchronize()
    ref = pipeline.gemm(op, lhs, rhs, T, Din, Dout, pl, pr, route=route, k=k, rows=rows, cols=cols)
    assert A.ROUTE_NAME[plan.route] == ref["route"]
    if ref["route"] != "BF16":
        v = A.workspace_views(ws, plan)
        if ref["idx"] is not None:
            assert np.array_equal(host(v["idx"]), ref["idx"])
        for key in ("a_codes", "a_scales", "b_codes", "b_scales"):
            assert np.array_equal(host(v[key]), ref[key]), key
    C32, C16 = host(c32), host(c16)
    if rows is not None:
        C32 = C32[np.ix_(rows, cols)]
        C16 = C16[np.ix_(rows, cols)]
    g = gamma_of(ref)
    check_f32(C32, ref["C"], g, f"{op} {ref['route']} f32")
    say("  " + describe(check_bf16(C16, ref["C"], g, f"{op} {ref['route']} bf16")))
    assert np.array_equal(C16, f32_to_bf16_rne(C32))
    return ref


FULL_CASES = [
    # op, T, Din, Dout, pl, pr, route, k
    ("FWD", 256, 512, 512, "C", "N", None, 64),
    ("FWD", 256, 512, 512, "C", "N", "OE_INNER", 16),
    ("FWD", 256, 512, 512, "C", "N", "MXFP4", 64),
    ("FWD", 300, 256, 200, "R", "N", None, 8),          # OE_LEFT (X rows)
    ("FWD", 300, 256, 200, "N", "R", None, 8),          # OE_RIGHT (W rows)
    ("FWD", 96, 64, 80, "R", "R", None, 8),             # BF16
    ("DGRAD", 512, 384, 256, "R", "N", None, 8),        # OE_LEFT (GY rows)
    ("DGRAD", 512, 384, 256, "N", "N", None, 64),       # IHT, W column-major
    ("DGRAD", 320, 192, 256, "N", "C", None, 8),        # OE_RIGHT (W cols)
    ("DGRAD", 320, 192, 256, "C", "N", "OE_INNER", 8),
    ("WGRAD", 512, 384, 256, "R", "C", None, 8),        # OE_RIGHT (X cols)
    ("WGRAD", 512, 384, 256, "C", "N", None, 8),        # OE_LEFT (GY cols)
    ("WGRAD", 416, 160, 96, "R", "N", "OE_INNER", 8),
    ("WGRAD", 128, 96, 64, "C", "C", None, 8),          # BF16 (ring kernel, both in place)
    # BF16 route, K % 128 == 0: the ring kernel on bf16 matrix cores; an
    # operand not contiguous along K is read across K in place, or from a
    # K-major copy when its row length is not a multiple of 8
    ("FWD", 300, 512, 200, "R", "R", None, 8),          # both contiguous, ragged tiles
    ("DGRAD", 520, 132, 384, "N", "N", "BF16", 8),      # W copied (rows of 132)
    ("DGRAD", 520, 136, 384, "N", "N", "BF16", 8),      # W in place
    ("WGRAD", 1024, 200, 72, "C", "C", None, 8),        # GY and X in place, split tile
    ("WGRAD", 512, 100, 96, "C", "C", None, 8),         # GY in place, X copied
    ("WGRAD", 512, 96, 100, "C", "C", None, 8),         # GY copied, X in place
    ("FWD", 300, 2048, 200, "N", "N", "BF16", 8),       # 2 tiles split along K in 4 parts
    ("FWD", 8192, 256, 200, "R", "R", None, 8),         # W copied across K (8192 rows of X)
    ("FWD", 200, 256, 8192, "R", "R", None, 8),         # X copied across K (8192 rows of W)
    ("FWD", 200, 160, 72, "R", "R", None, 8),           # K % 128 != 0: the tile kernel
    # K % 512 == 0: operands packed K-chunked for the main GEMM kernel
    ("FWD", 300, 1024, 200, "R", "N", None, 8),         # OE_LEFT, both rows quantized in rows
    ("DGRAD", 520, 136, 512, "N", "C", None, 8),        # OE_RIGHT, W quantized down columns
    ("WGRAD", 1024, 200, 72, "R", "C", None, 8),        # OE_RIGHT, both down columns
    ("WGRAD", 512, 96, 160, "C", "N", None, 8),         # OE_LEFT (GY columns)
    ("DGRAD", 300, 264, 1536, "N", "N", None, 64),      # IHT, ragged tiles
    # few tiles, long K: the main kernel splits each tile along K
    ("WGRAD", 4096, 200, 300, "R", "C", None, 8),       # OE_RIGHT, 2 parts
    ("FWD", 256, 8192, 520, "C", "N", "OE_INNER", 16),  # inner term, 4 parts
]


@pytest.mark.parametrize("case", FULL_CASES, ids=[str(c) for c in FULL_CASES])
def test_full_product(case):
    op, T, Din, Dout, pl, pr, route, k = case
    lhs, rhs = operands(op, T, Din, Dout, pl, pr, seed=T + Din)
    run_and_compare(op, lhs, rhs, T, Din, Dout, pl, pr, route, k)


# Long contractions with operands of 128 MiB and more that FOID does not
# scan: the outlier product over many K splits, ragged edges. Sampled
# outputs plus every outlier line.
LONG_K_CASES = [
    # op, T, Din, Dout, pl, pr, k
    ("WGRAD", 16384, 136, 4002, "R", "C", 40),    # OE_RIGHT, GY rows % 4 != 0
    ("WGRAD", 16416, 4096, 72, "C", "N", 64),     # OE_LEFT, X; K % 128 == 32, ROWS layout
    ("DGRAD", 256, 4096, 16384, "R", "N", 24),    # OE_LEFT, W down its columns
]


@pytest.mark.parametrize("case", LONG_K_CASES, ids=[str(c) for c in LONG_K_CASES])
def test_full_product_long_k(case):
    op, T, Din, Dout, pl, pr, k = case
    plan = A.adahop_gemm_plan(op, T, Din, Dout, pl, pr, None, k)
    lhs, rhs = operands(op, T, Din, Dout, pl, pr, seed=T + Din + k)
    route = A.ROUTE_NAME[plan.route]
    tensor, axis = oracle.scan_target(op, route)
    idx = oracle.foid(lhs if tensor == 0 else rhs, axis, k)
    rng = np.random.default_rng(T + k)
    rows = np.unique(np.concatenate([rng.choice(plan.m, 40, replace=False),
                                     idx if route == "OE_LEFT" else []]).astype(np.int64))
    cols = np.unique(np.concatenate([rng.choice(plan.n, min(40, plan.n), replace=False),
                                     idx if route == "OE_RIGHT" else []]).astype(np.int64))
    run_and_compare(op, lhs, rhs, T, Din, Dout, pl, pr, None, k, rows=rows, cols=cols)


# Degenerate inputs: all-zero operands (every FOID score 0, so the lowest
# indices win; zero codes and scale bytes; C = 0), constant operands (every
# score 0 again, nonzero products), and k equal to the number of candidate
# lines (the FP4 residual is all zero and C is the bf16 outlier product).
DEGENERATE_CASES = [
    # op, T, Din, Dout, pl, pr, route, k, fill
    ("WGRAD", 512, 200, 136, "R", "C", None, 16, "zeros"),
    ("DGRAD", 256, 320, 512, "R", "N", None, 8, "zeros"),
    ("FWD", 256, 512, 264, "C", "N", None, 64, "zeros"),
    ("WGRAD", 512, 96, 160, "R", "C", None, 32, "const"),
    ("FWD", 300, 256, 200, "R", "N", "OE_INNER", 16, "const"),
    ("WGRAD", 1024, 64, 200, "R", "C", None, 64, "planted"),      # k = all 64 of X's columns
    ("DGRAD", 96, 512, 1024, "R", "N", None, 96, "planted"),      # k = all 96 of GY's rows
]


@pytest.mark.parametrize("case", DEGENERATE_CASES, ids=[str(c) for c in DEGENERATE_CASES])
def test_full_product_degenerate(case):
    op, T, Din, Dout, pl, pr, route, k, fill = case
    if fill == "planted":
        lhs, rhs = operands(op, T, Din, Dout, pl, pr, seed=T + k)
    else:
        lhs, rhs = operands(op, T, Din, Dout, pl, pr, seed=1)
        # +0 is 0x0000; 1.5 is 0x3FC0 in bf16
        lhs = np.full_like(lhs, 0 if fill == "zeros" else 0x3FC0)
        rhs = np.full_like(rhs, 0 if fill == "zeros" else 0x3FC0)
    ref = run_and_compare(op, lhs, rhs, T, Din, Dout, pl, pr, route, k)
    if fill == "zeros":
        assert not np.any(ref["C"])
    if ref["idx"] is not None and fill != "planted":
        assert np.array_equal(ref["idx"], np.arange(k))


# FOID's selection in one launch with the quantization of the operand it
# does not scan (256-thread workgroups), one case per shape of the selection:
# a lone final level, first-level chunks of 256, 512 and 1024 candidates (1,
# 2 and 4 per thread), and k = 200; and with that operand quantized down its
# columns or along its rows. The scanned operand holds 0/1 values
# (scores take few distinct values: the k-th is tied) with k/2 lines x3, so
# the tie-break by index decides the boundary; indices, codes and scales
# bit-exact, the output to the product bar.
BESIDE_CASES = [
    # op, T, Din, Dout, pattern pair, route, k
    ("WGRAD", 256, 1000, 128, "R", "C", "OE_RIGHT", 100),   # 1000 of X's columns: the final level alone
    ("WGRAD", 256, 3000, 128, "R", "C", "OE_RIGHT", 64),    # 12 chunks of 256, the last ragged
    ("WGRAD", 256, 6000, 128, "R", "C", "OE_RIGHT", 64),    # 12 chunks of 512
    ("WGRAD", 256, 9000, 128, "R", "C", "OE_RIGHT", 64),    # 9 chunks of 1024
    ("WGRAD", 256, 5000, 128, "R", "C", "OE_RIGHT", 200),   # 5 chunks of 1024, 1000 survivors
    ("DGRAD", 3000, 256, 512, "R", "N", "OE_LEFT", 32),     # GY's rows, 12 chunks of 256
    # the other operand quantized along its rows (row-direction tiles)
    ("FWD", 3000, 256, 512, "R", "N", "OE_LEFT", 32),       # X's rows; W along its rows
    ("FWD", 512, 256, 5000, "N", "R", "OE_RIGHT", 64),      # W's rows, 10 chunks of 512; X along its rows
    ("DGRAD", 512, 3000, 256, "N", "C", "OE_RIGHT", 64),    # W's columns; GY along its rows
    ("FWD", 300, 1024, 200, "R", "N", "OE_LEFT", 8),        # a lone final level
]


@pytest.mark.parametrize("case", BESIDE_CASES, ids=[str(c) for c in BESIDE_CASES])
def test_foid_beside_other_quantization(case):
    op, T, Din, Dout, pl, pr, route, k = case
    rng = np.random.default_rng(T + Din + k)
    shapes = {"FWD": ((T, Din), (Dout, Din)), "DGRAD": ((T, Dout), (Dout, Din)),
              "WGRAD": ((T, Dout), (T, Din))}[op]
    scan, oaxis = oracle.scan_target(op, route)
    axis = 0 if oaxis == oracle.ROWS else 1
    ops = []
    for t, shape in enumerate(shapes):
        if t != scan:
            ops.append(rand_bf16(rng, shape))
            continue
        v = rng.integers(0, 2, size=shape).astype(np.float32)
        lines = rng.choice(shape[axis], k // 2, replace=False)
        if axis == 0:
            v[lines, :] *= 3.0
        else:
            v[:, lines] *= 3.0
        ops.append(f32_to_bf16_rne(v))
    ref = run_and_compare(op, ops[0], ops[1], T, Din, Dout, pl, pr, route, k)
    assert set(lines.tolist()) <= set(ref["idx"].tolist())


# The outlier product formed in the quantization of the operand FOID does
# not scan (adahop_gemm_ex with oe_in_quant): that operand's quantized codes
# and scales, the indices and the gathered lines bit-exact, the output to
# the product bar (the outlier product's sum is added before the single
# rounding). K-chunked and row layouts, a ragged last group of tiles and a
# ragged column tile, element loads (a row length not a multiple of 4), k
# from 1 to 64 with partial line blocks.
ONE_READ_CASES = [
    # op, T, Din, Dout, pattern pair, route, k
    ("WGRAD", 4096, 768, 512, "R", "C", "OE_RIGHT", 16),    # GY quantized with the product, 8 groups
    ("WGRAD", 4000, 300, 200, "C", "N", "OE_LEFT", 64),     # X with the product, [k][n]; K % 128 == 32
    ("DGRAD", 777, 300, 2048, "R", "N", "OE_LEFT", 40),     # W with the product; k = 40
    ("WGRAD", 16384, 136, 4002, "R", "C", "OE_RIGHT", 1),   # GY rows of 4002: element loads
    ("WGRAD", 8192, 6400, 256, "R", "C", "OE_RIGHT", 64),   # X scanned by columns, operands above 96 MB
]


@pytest.mark.parametrize("case", ONE_READ_CASES, ids=[str(c) for c in ONE_READ_CASES])
def test_full_product_oe_in_quant(case):
    op, T, Din, Dout, pl, pr, route, k = case
    lhs, rhs = operands(op, T, Din, Dout, pl, pr, seed=T + Din + Dout + k)
    plan = A.adahop_gemm_plan(op, T, Din, Dout, pl, pr, route, k)
    rows = cols = None
    if plan.m * plan.n > 1 << 20:
        rng = np.random.default_rng(T + k)
        rows = np.unique(rng.choice(plan.m, min(48, plan.m), replace=False))
        cols = np.unique(rng.choice(plan.n, min(48, plan.n), replace=False))
        tensor, axis = oracle.scan_target(op, route)
        idx = oracle.foid(lhs if tensor == 0 else rhs, axis, k)
        if route == "OE_LEFT":
            rows = np.unique(np.concatenate([rows, idx[:8]]))
        else:
            cols = np.unique(np.concatenate([cols, idx[:8]]))
        rows, cols = rows.astype(np.int64), cols.astype(np.int64)
    run_and_compare(op, lhs, rhs, T, Din, Dout, pl, pr, route, k, rows=rows, cols=cols,
                    oe_in_quant=True)


def test_deterministic_reruns():
    # K = 4096 over 6 tiles: the K-split path, whose parts are added in order.
    op, T, Din, Dout = "WGRAD", 4096, 768, 512
    lhs, rhs = operands(op, T, Din, Dout, "R", "C", 3)
    L, R = dev_bf16(lhs), dev_bf16(rhs)
    say("determinism")
    a = A.adahop_gemm(op, L, R, "R", "C", None, 16)
    b = A.adahop_gemm(op, L, R, "R", "C", None, 16)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("T", [512, 2048], ids=["separate-outlier-kernel", "outlier-items-in-gemm"])
def test_stage_events_record(T):
    # The timed call (an event between the GEMM's main kernel and its tail)
    # gives the untimed call's output bit for bit, with ordered events; at
    # T = 2048 the outlier product runs inside the main kernel and the tail
    # holds its scatter.
    op, Din, Dout = "WGRAD", 384, 256
    lhs, rhs = operands(op, T, Din, Dout, "R", "C", 4)
    L, R = dev_bf16(lhs), dev_bf16(rhs)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(A.STAGE_EVENTS)]
    say("stage events", T)
    timed = A.adahop_gemm(op, L, R, "R", "C", None, 8, stage_events=ev)
    plain = A.adahop_gemm(op, L, R, "R", "C", None, 8)
    torch.cuda.synchronize()
    assert torch.equal(timed.view(torch.int16), plain.view(torch.int16))
    times = [ev[i].elapsed_time(ev[i + 1]) for i in range(A.STAGE_EVENTS - 1)]
    assert all(t >= 0 for t in times)


@pytest.mark.parametrize("case", [("FWD", 8192, 256, 200), ("WGRAD", 512, 100, 96)],
                         ids=["fwd-copy-across", "wgrad-in-place-and-copy"])
def test_stage_events_bf16_route(case):
    # The timed call on the BF16 route (its copies in the operand stages)
    # gives the untimed call's output bit for bit, with ordered events.
    op, T, Din, Dout = case
    lhs, rhs = operands(op, T, Din, Dout, "N", "N", 5)
    L, R = dev_bf16(lhs), dev_bf16(rhs)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(A.STAGE_EVENTS)]
    say("stage events BF16", case)
    timed = A.adahop_gemm(op, L, R, "N", "N", "BF16", 1, stage_events=ev)
    plain = A.adahop_gemm(op, L, R, "N", "N", "BF16", 1)
    torch.cuda.synchronize()
    assert torch.equal(timed.view(torch.int16), plain.view(torch.int16))
    times = [ev[i].elapsed_time(ev[i + 1]) for i in range(A.STAGE_EVENTS - 1)]
    assert all(t >= 0 for t in times)
