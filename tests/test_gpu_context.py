"""The saved forward context on the GPU (adahop_ctx_save, then
adahop_gemm_wgrad_ctx) against the oracle's context and against the plain
weight gradient: the kept indices, codes, scales and lines bit-exact; the
weight gradient from the context bit-identical to adahop_gemm's from X (fp32
and bf16 outputs, whole output) and within the GEMM bar of the oracle's."""
import numpy as np
import pytest
import torch

import mxfp4_precision_gemms_amd as A
from oracle import pipeline
from parity import check_bf16, check_f32, describe, gamma_of
from synth import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def dev_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)


def host(t):
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.int16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def check_context(X, Dout, pg, px, route, k):
    T, Din = X.shape
    plan = A.adahop_ctx_plan(T, Din, Dout, pg, px, route, k)
    ctx = A.adahop_ctx_save(dev_bf16(X), Dout, pg, px, route, k)
    torch.cuda.synchronize()
    ref = pipeline.forward_context(X, pg, px, route, k)
    assert A.ROUTE_NAME[plan.route] == ref["route"]
    v = A.ctx_views(ctx, plan)
    if ref["idx"] is None:
        assert v["idx"] is None and v["lines"] is None
    else:
        assert np.array_equal(host(v["idx"]), ref["idx"])
        assert np.array_equal(host(v["lines"]), ref["lines"])
    assert np.array_equal(host(v["codes"]), ref["codes"])
    assert np.array_equal(host(v["scales"]), ref["scales"])
    return plan, ctx, ref


SMALL = [
    # T, Din, Dout, pat GY, pat X, route, k
    (256, 96, 64, "R", "C", None, 4),          # OE_RIGHT, ROWS layout (T % 512 != 0)
    (1024, 384, 256, "R", "C", None, 8),       # OE_RIGHT, K-chunked
    (1024, 384, 256, "N", "N", None, 8),       # IHT
    (512, 200, 136, "R", "N", "MXFP4", 8),     # plain MXFP4, ragged tiles
    (4096, 520, 300, "R", "C", None, 16),      # split tail, 2 K-parts
]


@pytest.mark.parametrize("case", SMALL, ids=[str(c) for c in SMALL])
def test_context_small(case):
    T, Din, Dout, pg, px, route, k = case
    say("context", case)
    wl_x = W.TensorSpec("X", T, Din, px if px != "N" else "N", max(1, Din // 100) if px != "N" else 0, 50.0)
    wl_gy = W.TensorSpec("GY", T, Dout, pg if pg != "N" else "N", max(1, T // 200) if pg != "N" else 0, 100.0)
    X, GY = wl_x.make(1), wl_gy.make(1)
    plan, ctx, cref = check_context(X, Dout, pg, px, route, k)
    G = dev_bf16(GY)
    outs = {}
    for dt in (torch.float32, torch.bfloat16):
        a = A.adahop_gemm_wgrad_ctx(G, ctx, Din, pg, px, route, k, out_dtype=dt)
        b = A.adahop_gemm("WGRAD", G, dev_bf16(X), pg, px, route, k, out_dtype=dt)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32) if dt == torch.float32 else a.view(torch.int16),
                           b.view(torch.int32) if dt == torch.float32 else b.view(torch.int16))
        outs[dt] = host(a)
    ref = pipeline.wgrad_from_context(GY, cref, T, Din, Dout, pg)
    g = gamma_of(ref)
    check_f32(outs[torch.float32], ref["C"], g, f"{case} f32")
    say("  " + describe(check_bf16(outs[torch.bfloat16], ref["C"], g, f"{case} bf16")))


FULL = [("l31_8b_oproj_triplet", 8), ("l31_8b_down_wgrad", None)]


@pytest.mark.parametrize("name,bs", FULL, ids=[f"{n}-{b}" for n, b in FULL])
def test_context_full_size(name, bs):
    wl = W.l31_8b_oproj_triplet(bs) if bs else W.l31_8b_down_wgrad()
    call = [c for c in wl.calls if c.op == "WGRAD"][0]
    T, Din, Dout = wl.T, wl.Din, wl.Dout
    say("context full size", wl.name, (T, Din, Dout))
    X = wl.tensors[call.rhs].make(0)
    GY = wl.tensors[call.lhs].make(0)
    plan, ctx, cref = check_context(X, Dout, call.pat_lhs, call.pat_rhs, call.route, call.k)
    assert A.ROUTE_NAME[plan.route] == "OE_RIGHT" and plan.layout == A.LAYOUT_KCHUNK
    say(f"  context {plan.ctx_bytes / 2**20:.1f} MiB for X of {2 * T * Din / 2**20:.1f} MiB "
        f"({2 * T * Din / plan.ctx_bytes:.2f}x)")
    G, Xd = dev_bf16(GY), dev_bf16(X)
    a = A.adahop_gemm_wgrad_ctx(G, ctx, Din, call.pat_lhs, call.pat_rhs, call.route, call.k,
                                out_dtype=torch.float32)
    b = A.adahop_gemm("WGRAD", G, Xd, call.pat_lhs, call.pat_rhs, call.route, call.k,
                      out_dtype=torch.float32)
    a16 = A.adahop_gemm_wgrad_ctx(G, ctx, Din, call.pat_lhs, call.pat_rhs, call.route, call.k)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(a.to(torch.bfloat16).view(torch.int16), a16.view(torch.int16))
