"""Seeded random whole products against the oracle: every op, pattern pair
and route; small sizes (1 to about 700, the contraction a multiple of 32,
every output checked) and larger ones (up to ~3000 with the contraction up
to 8192, sampled outputs plus outlier lines), outlier ranks from 1 to the
number of candidate lines. Bit-exact route, FOID indices, codes and scales;
the GEMM bar on the output (tests/parity.py). Also products with the outer
outlier product formed in the other operand's quantization (oe_in_quant)."""
import numpy as np
import pytest

import mxfp4_precision_gemms_amd as A
from test_gpu_parity import operands, run_and_compare

pytestmark = pytest.mark.gpu

OPS = ("FWD", "DGRAD", "WGRAD")
PATS = ("N", "R", "C")
ROUTES = (None, None, None, "IHT", "MXFP4", "OE_LEFT", "OE_RIGHT", "OE_INNER", "BF16")


def random_case(i):
    rng = np.random.default_rng(9000 + i)
    op = OPS[i % 3]
    dims = [int(rng.integers(1, 700)) for _ in range(3)]
    T, Din, Dout = dims
    # the contraction length is a multiple of 32
    c = {"FWD": 1, "DGRAD": 2, "WGRAD": 0}[op]
    dims[c] = 32 * int(rng.integers(1, 22))
    T, Din, Dout = dims
    pl, pr = PATS[int(rng.integers(0, 3))], PATS[int(rng.integers(0, 3))]
    route = ROUTES[int(rng.integers(0, len(ROUTES)))]
    plan = A.adahop_gemm_plan(op, T, Din, Dout, pl, pr, route, 1)
    k = 1
    if plan.scan_tensor >= 0:
        shape = {"FWD": ((T, Din), (Dout, Din)), "DGRAD": ((T, Dout), (Dout, Din)),
                 "WGRAD": ((T, Dout), (T, Din))}[op][plan.scan_tensor]
        ncand = shape[0] if plan.scan_axis == 0 else shape[1]
        k = int(rng.integers(1, min(ncand, 128) + 1))
    return op, T, Din, Dout, pl, pr, route, k


CASES = [random_case(i) for i in range(36)]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_random_product(case):
    op, T, Din, Dout, pl, pr, route, k = case
    lhs, rhs = operands(op, T, Din, Dout, pl, pr, seed=T * 7 + Din * 3 + Dout)
    run_and_compare(op, lhs, rhs, T, Din, Dout, pl, pr, route, k)


ROUTES_LARGE = (None, None, "IHT", "MXFP4", "OE_LEFT", "OE_RIGHT", "OE_INNER")


def random_large_case(i):
    """Sizes up to ~3000 with the contraction up to 8192 (K-chunked packing,
    K splits of the last round of tiles, ragged tiles), ranks up to 256."""
    rng = np.random.default_rng(50000 + i)
    op = OPS[i % 3]
    dims = [int(rng.integers(1, 3000)) for _ in range(3)]
    c = {"FWD": 1, "DGRAD": 2, "WGRAD": 0}[op]
    dims[c] = int(rng.choice([512, 1024, 1536, 2048, 4096, 8192, 128 * int(rng.integers(1, 64))]))
    T, Din, Dout = dims
    pl, pr = PATS[int(rng.integers(0, 3))], PATS[int(rng.integers(0, 3))]
    route = ROUTES_LARGE[int(rng.integers(0, len(ROUTES_LARGE)))]
    plan = A.adahop_gemm_plan(op, T, Din, Dout, pl, pr, route, 1)
    k = 1
    if plan.scan_tensor >= 0:
        shape = {"FWD": ((T, Din), (Dout, Din)), "DGRAD": ((T, Dout), (Dout, Din)),
                 "WGRAD": ((T, Dout), (T, Din))}[op][plan.scan_tensor]
        ncand = shape[0] if plan.scan_axis == 0 else shape[1]
        k = int(rng.integers(1, min(ncand, 256) + 1))
    return op, T, Din, Dout, pl, pr, route, k


LARGE_CASES = [random_large_case(i) for i in range(24)]


@pytest.mark.parametrize("case", LARGE_CASES, ids=[str(c) for c in LARGE_CASES])
def test_random_large_product(case):
    import oracle
    op, T, Din, Dout, pl, pr, route, k = case
    lhs, rhs = operands(op, T, Din, Dout, pl, pr, seed=T + Din + Dout)
    plan = A.adahop_gemm_plan(op, T, Din, Dout, pl, pr, route, k)
    rng = np.random.default_rng(T * Din)
    rows = np.unique(rng.choice(plan.m, min(24, plan.m), replace=False))
    cols = np.unique(rng.choice(plan.n, min(24, plan.n), replace=False))
    rname = A.ROUTE_NAME[plan.route]
    if rname in ("OE_LEFT", "OE_RIGHT"):
        # every sampled set also holds outlier lines, where the scatter-add lands
        tensor, axis = oracle.scan_target(op, rname)
        idx = oracle.foid(lhs if tensor == 0 else rhs, axis, k)
        if rname == "OE_LEFT":
            rows = np.unique(np.concatenate([rows, idx[:8]]))
        else:
            cols = np.unique(np.concatenate([cols, idx[:8]]))
    run_and_compare(op, lhs, rhs, T, Din, Dout, pl, pr, route, k,
                    rows=rows.astype(np.int64), cols=cols.astype(np.int64))


def random_bf16_case(i):
    """The BF16 route: sizes up to ~1500 with ragged tiles, the contraction a
    multiple of 128 (the ring kernel; operands stored across K read in place
    when their rows are a multiple of 8 elements, else copied) or, one case
    in four, only of 32 (the tile kernel)."""
    rng = np.random.default_rng(70000 + i)
    op = OPS[i % 3]
    dims = [int(rng.integers(1, 1500)) for _ in range(3)]
    c = {"FWD": 1, "DGRAD": 2, "WGRAD": 0}[op]
    dims[c] = 32 * int(rng.integers(1, 64)) if i % 4 == 3 else 128 * int(rng.integers(1, 24))
    for d in range(3):
        if d != c and rng.random() < 0.5:
            dims[d] = 8 * max(1, dims[d] // 8)      # rows a multiple of 8: read in place
    T, Din, Dout = dims
    return op, T, Din, Dout


BF16_CASES = [random_bf16_case(i) for i in range(16)]


@pytest.mark.parametrize("case", BF16_CASES, ids=[str(c) for c in BF16_CASES])
def test_random_bf16_route(case):
    op, T, Din, Dout = case
    lhs, rhs = operands(op, T, Din, Dout, "N", "N", seed=T + 2 * Din + 3 * Dout)
    plan = A.adahop_gemm_plan(op, T, Din, Dout, "N", "N", "BF16", 1)
    rows = cols = None
    if plan.m * plan.n > 512 * 512:
        rng = np.random.default_rng(T * Dout)
        rows = np.unique(rng.choice(plan.m, min(48, plan.m), replace=False)).astype(np.int64)
        cols = np.unique(rng.choice(plan.n, min(48, plan.n), replace=False)).astype(np.int64)
    run_and_compare(op, lhs, rhs, T, Din, Dout, "N", "N", "BF16", 1, rows=rows, cols=cols)


def random_one_read_case(i):
    """A seeded OE_LEFT / OE_RIGHT product whose other operand is quantized
    down its columns (DGRAD's W, either WGRAD operand), run with the outlier
    product formed in that operand's quantization (oe_in_quant): sizes up to
    ~2000 with the contraction up to 8192, k from 1 to 64."""
    rng = np.random.default_rng(90000 + i)
    while True:
        # odd cases OE_RIGHT (a weight gradient's X columns), even ones OE_LEFT
        op = "WGRAD" if i % 2 else ("DGRAD", "WGRAD")[int(rng.integers(0, 2))]
        dims = [int(rng.integers(1, 2000)) for _ in range(3)]
        c = {"DGRAD": 2, "WGRAD": 0}[op]
        dims[c] = int(rng.choice([512, 2048, 4096, 8192, 32 * int(rng.integers(1, 128))]))
        T, Din, Dout = dims
        pl, pr = PATS[int(rng.integers(0, 3))], PATS[int(rng.integers(0, 3))]
        route = "OE_RIGHT" if i % 2 else "OE_LEFT"
        plan = A.adahop_gemm_plan(op, T, Din, Dout, pl, pr, route, 1)
        shape = {"DGRAD": ((T, Dout), (Dout, Din)), "WGRAD": ((T, Dout), (T, Din))}[op][plan.scan_tensor]
        ncand = shape[0] if plan.scan_axis == 0 else shape[1]
        k = int(rng.integers(1, min(ncand, 64) + 1))
        if A.adahop_gemm_plan(op, T, Din, Dout, pl, pr, route, k, oe_in_quant=True).oe_in_quant:
            return op, T, Din, Dout, pl, pr, route, k


ONE_READ_CASES = [random_one_read_case(i) for i in range(10)]


@pytest.mark.parametrize("case", ONE_READ_CASES, ids=[str(c) for c in ONE_READ_CASES])
def test_random_one_read_product(case):
    import oracle
    op, T, Din, Dout, pl, pr, route, k = case
    lhs, rhs = operands(op, T, Din, Dout, pl, pr, seed=T + 5 * Din + 7 * Dout)
    plan = A.adahop_gemm_plan(op, T, Din, Dout, pl, pr, route, k)
    rng = np.random.default_rng(T * Dout + k)
    rows = np.unique(rng.choice(plan.m, min(32, plan.m), replace=False))
    cols = np.unique(rng.choice(plan.n, min(32, plan.n), replace=False))
    # every sampled set also holds outlier lines, where the product lands
    tensor, axis = oracle.scan_target(op, route)
    idx = oracle.foid(lhs if tensor == 0 else rhs, axis, k)
    if route == "OE_LEFT":
        rows = np.unique(np.concatenate([rows, idx[:8]]))
    else:
        cols = np.unique(np.concatenate([cols, idx[:8]]))
    run_and_compare(op, lhs, rhs, T, Din, Dout, pl, pr, route, k,
                    rows=rows.astype(np.int64), cols=cols.astype(np.int64), oe_in_quant=True)
