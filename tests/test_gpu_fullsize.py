"""GPU vs oracle parity at the full sizes of the synthetic Llama workloads,
through adahop_gemm with the same shapes, routes and launch configuration the
benchmark times.

Bit-exact over the whole call: route, FOID indices, MXFP4 codes and scales of
both operands, gathered bf16 lines. The output is compared on a sampled grid
of rows x columns (seeded random lines plus outlier lines where the route
scatters into C), which the oracle computes element by element in fp64, with
the GEMM bar of tests/parity.py; over the whole output, the bf16 result must
equal the round-to-nearest-even of the same call's fp32 result (one rounding,
checked on the device).
"""
import numpy as np
import pytest
import torch

import mxfp4_precision_gemms_amd as A
import oracle
from oracle import pipeline
from parity import check_bf16, check_f32, describe, gamma_of
from synth import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NONE = (1 << 64) - 1


def say(*a):
    print(*a, flush=True)


def dev_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def sample_lines(rng, dim, count, must=None, n_must=16):
    """`count` distinct random lines of [0, dim), plus up to n_must of `must`."""
    pick = rng.choice(dim, size=min(count, dim), replace=False)
    if must is not None and len(must):
        pick = np.concatenate([pick, rng.choice(must, size=min(n_must, len(must)), replace=False)])
    return np.unique(pick).astype(np.int64)


CALLS = [
    # workload builder, call index
    ("tiny_fwd", 0), ("tiny_fwd", 1),
    ("l32_1b_up_fwd", 0),
    ("l31_8b_down_wgrad", 0),
    ("l31_8b_gateup_fwd_dgrad", 0), ("l31_8b_gateup_fwd_dgrad", 1),
    ("l31_8b_oproj_triplet_bs1", 0), ("l31_8b_oproj_triplet_bs1", 1),
    ("l31_8b_oproj_triplet_bs1", 2),
    ("l31_8b_oproj_triplet_bs16", 0), ("l31_8b_oproj_triplet_bs16", 1),
    ("l31_8b_oproj_triplet_bs16", 2),
    ("l31_8b_oproj_triplet_bs2", 0), ("l31_8b_oproj_triplet_bs2", 1),
    ("l31_8b_oproj_triplet_bs2", 2),
    ("l31_8b_oproj_triplet_bs4", 0), ("l31_8b_oproj_triplet_bs4", 1),
    ("l31_8b_oproj_triplet_bs4", 2),
    ("l31_8b_oproj_triplet_bs8", 0), ("l31_8b_oproj_triplet_bs8", 1),
    ("l31_8b_oproj_triplet_bs8", 2),
]


def workload(name):
    if name.startswith("l31_8b_oproj_triplet_bs"):
        return W.l31_8b_oproj_triplet(int(name.rsplit("bs", 1)[1]))
    return getattr(W, name)()


@pytest.mark.parametrize("name,ci", CALLS, ids=[f"{n}-{c}" for n, c in CALLS])
def test_full_size_call(name, ci):
    full_size(name, ci)


# The outer outlier product formed in the quantization of the operand FOID
# does not scan (adahop_gemm_ex, oe_in_quant), at the benchmark's sizes.
ONE_READ_CALLS = [("l31_8b_down_wgrad", 0), ("l31_8b_oproj_triplet_bs1", 1),
                  ("l31_8b_oproj_triplet_bs1", 2), ("l31_8b_oproj_triplet_bs16", 2)]


@pytest.mark.parametrize("name,ci", ONE_READ_CALLS, ids=[f"{n}-{c}" for n, c in ONE_READ_CALLS])
def test_full_size_call_oe_in_quant(name, ci):
    full_size(name, ci, oe_in_quant=True)


def full_size(name, ci, oe_in_quant=False):
    wl = workload(name)
    call = wl.calls[ci]
    op, T, Din, Dout = call.op, wl.T, wl.Din, wl.Dout
    say("full size", name, ci, op, (T, Din, Dout), call.pat_lhs + call.pat_rhs, call.route, call.k,
        "oe_in_quant" if oe_in_quant else "")
    lhs = wl.tensors[call.lhs].make(0)
    rhs = wl.tensors[call.rhs].make(0)
    plan = A.adahop_gemm_plan(op, T, Din, Dout, call.pat_lhs, call.pat_rhs, call.route, call.k,
                              oe_in_quant)
    assert plan.oe_in_quant == (1 if oe_in_quant else 0)
    m, n, K = plan.m, plan.n, plan.K
    ws = torch.empty(max(plan.ws_bytes, 1), dtype=torch.uint8, device=DEV)
    L, R = dev_bf16(lhs), dev_bf16(rhs)
    c32 = A.adahop_gemm(op, L, R, call.pat_lhs, call.pat_rhs, call.route, call.k,
                        out_dtype=torch.float32, ws=ws, oe_in_quant=oe_in_quant)
    torch.cuda.synchronize()
    v = A.workspace_views(ws, plan)
    got = {key: (host(v[key]) if v[key] is not None else None)
           for key in ("idx", "a_codes", "a_scales", "b_codes", "b_scales")}
    lines = {}
    for key, off in (("a_gathered", plan.off_lhs_lines), ("b_gathered", plan.off_rhs_lines)):
        lines[key] = None if off == NONE else off
    c16 = A.adahop_gemm(op, L, R, call.pat_lhs, call.pat_rhs, call.route, call.k,
                        out_dtype=torch.bfloat16, ws=ws, oe_in_quant=oe_in_quant)
    # One rounding, over the whole output.
    assert torch.equal(c32.to(torch.bfloat16).view(torch.int16), c16.view(torch.int16))
    del L, R

    rng = np.random.default_rng(1000 + ci)
    tiny = m * n <= 512 * 512
    route = call.route or oracle.route(op, call.pat_lhs, call.pat_rhs)
    assert A.ROUTE_NAME[plan.route] == route
    idx = None
    if route in ("OE_LEFT", "OE_RIGHT"):
        tensor, axis = oracle.scan_target(op, route)
        idx = oracle.foid(lhs if tensor == 0 else rhs, axis, call.k)
    if tiny:
        rows, cols = np.arange(m), np.arange(n)
    else:
        rows = sample_lines(rng, m, 48, idx if route == "OE_LEFT" else None)
        cols = sample_lines(rng, n, 48, idx if route == "OE_RIGHT" else None)
    ref = pipeline.gemm(op, lhs, rhs, T, Din, Dout, call.pat_lhs, call.pat_rhs,
                        route=call.route, k=call.k, rows=rows, cols=cols)

    assert ref["route"] == route
    if ref["idx"] is not None:
        assert np.array_equal(got["idx"], ref["idx"])
    for key in ("a_codes", "a_scales", "b_codes", "b_scales"):
        assert np.array_equal(got[key], ref[key]), key
    for key, off in lines.items():
        if off is None:
            continue
        g = ref[key]
        dev = host(ws[off:off + 2 * g.size].view(torch.int16)).view(np.uint16)
        assert np.array_equal(dev, np.ascontiguousarray(g).ravel()), key

    C32 = host(c32[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)])
    C16 = host(c16[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)])
    g = gamma_of(ref)
    rel = check_f32(C32, ref["C"], g, f"{name} {op} f32")
    st = check_bf16(C16, ref["C"], g, f"{name} {op} bf16")
    say(f"  {route} m={m} n={n} K={K}: sampled {rows.size}x{cols.size}, rel f32 {rel:.2e}; "
        + describe(st))


BF16_CALLS = [
    ("l31_8b_down_wgrad", 0),                                   # WGRAD: GY and X transposed
    ("l31_8b_gateup_fwd_dgrad", 0), ("l31_8b_gateup_fwd_dgrad", 1),   # FWD; DGRAD: W transposed
    ("l31_8b_oproj_triplet_bs1", 0),                            # 1024 x 4096 x 4096
]


@pytest.mark.parametrize("name,ci", BF16_CALLS, ids=[f"{n}-{c}" for n, c in BF16_CALLS])
def test_full_size_bf16_route(name, ci):
    # The same products forced onto the BF16 route (the ring kernel on bf16
    # matrix cores at these sizes), as the benchmark's --route BF16 times
    # them: sampled outputs against the oracle's fp64 product, and one
    # rounding over the whole output.
    wl = workload(name)
    call = wl.calls[ci]
    op, T, Din, Dout = call.op, wl.T, wl.Din, wl.Dout
    say("full size BF16 route", name, ci, op, (T, Din, Dout))
    lhs = wl.tensors[call.lhs].make(0)
    rhs = wl.tensors[call.rhs].make(0)
    plan = A.adahop_gemm_plan(op, T, Din, Dout, call.pat_lhs, call.pat_rhs, "BF16", 1)
    m, n, K = plan.m, plan.n, plan.K
    assert K % 128 == 0
    ws = torch.empty(max(plan.ws_bytes, 1), dtype=torch.uint8, device=DEV)
    L, R = dev_bf16(lhs), dev_bf16(rhs)
    c32 = A.adahop_gemm(op, L, R, call.pat_lhs, call.pat_rhs, "BF16", 1,
                        out_dtype=torch.float32, ws=ws)
    c16 = A.adahop_gemm(op, L, R, call.pat_lhs, call.pat_rhs, "BF16", 1,
                        out_dtype=torch.bfloat16, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(c32.to(torch.bfloat16).view(torch.int16), c16.view(torch.int16))
    del L, R
    rng = np.random.default_rng(2000 + ci)
    rows, cols = sample_lines(rng, m, 48), sample_lines(rng, n, 48)
    ref = pipeline.gemm(op, lhs, rhs, T, Din, Dout, call.pat_lhs, call.pat_rhs,
                        route="BF16", k=1, rows=rows, cols=cols)
    assert ref["route"] == "BF16"
    C32 = host(c32[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)])
    C16 = host(c16[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)])
    g = gamma_of(ref)
    rel = check_f32(C32, ref["C"], g, f"{name} {op} BF16 f32")
    st = check_bf16(C16, ref["C"], g, f"{name} {op} BF16 bf16")
    say(f"  BF16 m={m} n={n} K={K}: sampled {rows.size}x{cols.size}, rel f32 {rel:.2e}; "
        + describe(st))
