"""Benchmark of one AdaHOP product (FOID + IHT + MXFP4 quantization + fused
FP4/bf16 GEMM + scatter-add) on one MI355X.

Default workload: the Llama3.1-8B down_proj weight gradient dW = GY^T X over
32768 tokens (seq 4096 x batch 8), GY [32768,4096] Row-wise (0.5% of rows
x100), X [32768,14336] Column-wise (1% of columns x50): RC pair -> OE-Right
with rank 64, i.e. every stage of the path runs. A step is one adahop_gemm
call on inputs already resident in HBM.

Prints one JSON line: effective TFLOP/s (2 m n K / wall time of the call),
ms per call, per-stage times from HIP events recorded by the library on the
call's stream, the roofline of the dominant kernel (the fused GEMM) and the
oracle timed on the host's cores on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

`--rank-sweep` prints instead the latency and error of the product at
outlier ranks 0-256 and in plain MXFP4 (the pages' variant study, Fig. 10).
`--route NAME` times the workload's product on another route, e.g. BF16
(the all-bf16 route; its roofline is then the bf16 GEMM's, against the bf16
peak).
"""
import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("effective TFLOPS per AdaHOP GEMM (FOID+IHT+quant+GEMM+OE) and % MXFP4 MFMA peak")
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense MXFP4 matrix-core peak
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0


def workloads():
    from synth import workloads as W
    out = {"l8b_down_wgrad": (W.l31_8b_down_wgrad(), 0)}
    g = W.l31_8b_gateup_fwd_dgrad()
    out["l8b_gateup_fwd"] = (g, 0)
    out["l8b_gateup_dgrad"] = (g, 1)
    out["l1b_up_fwd"] = (W.l32_1b_up_fwd(), 0)
    out["tiny_fwd"] = (W.tiny_fwd(), 0)
    for bs in (1, 2, 4, 8, 16):
        t = W.l31_8b_oproj_triplet(bs)
        for i, name in enumerate(("fwd", "dgrad", "wgrad")):
            out[f"l8b_oproj_bs{bs}_{name}"] = (t, i)
    return out


# HBM traffic of the GEMM kernel comes from rocprofv3 FETCH_SIZE / WRITE_SIZE
# passes (recorded with the copy-kernel calibration in this summary); it is
# reported only while the kernel source is byte-identical to the one counted.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_mx_ring_l8b_down_wgrad_traffic.md")
TRAFFIC_SUMMARY_BF16 = os.path.join(ROOT, "profiles", "bf16_ring_l8b_down_wgrad_traffic.md")


def measured_traffic(workload_name, summary=TRAFFIC_SUMMARY):
    """(bytes per launch or None, note)."""
    try:
        with open(summary) as f:
            text = f.read()
    except OSError:
        return None, "no counter summary"
    m = re.search(r"^traffic-record: (\{.*\})$", text, re.M)
    if not m:
        return None, "no traffic record in the counter summary"
    rec = json.loads(m.group(1))
    if rec["workload"] != workload_name:
        return None, "counters were taken on another workload"
    with open(os.path.join(ROOT, rec["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
            return None, "kernel source changed since the counters were taken"
    fetch = rec["fetch_kib"] * 1024 * rec["fetch_scale"]
    write = rec["write_kib"] * 1024 * rec["write_scale"]
    return fetch + write, (f"FETCH_SIZE {rec['fetch_kib']} KiB x{rec['fetch_scale']} + WRITE_SIZE "
                           f"{rec['write_kib']} KiB x{rec['write_scale']} per launch")


def gemm_dims(op, T, Din, Dout):
    return {"FWD": (T, Dout, Din), "DGRAD": (T, Din, Dout), "WGRAD": (Dout, Din, T)}[op]


def cpu_baseline(op, lhs, rhs, T, Din, Dout, call, m, n, K, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample of the same call,
    extrapolated to the full call: FOID in full; zero+IHT+quantization of
    both operands on a slab of contraction blocks (scaled by K / slab); the
    fp64 product of the dequantized operands on an output tile over that
    slab (scaled by m n K / (tile x slab)); the outlier product is inside the
    residual-product estimate's margin and is not timed separately."""
    import numpy as np

    import oracle

    t_all = time.perf_counter()
    route = call.route or oracle.route(op, call.pat_lhs, call.pat_rhs)
    t0 = time.perf_counter()
    idx = None
    if route in ("OE_LEFT", "OE_RIGHT", "OE_INNER"):
        tensor, axis = oracle.scan_target(op, route)
        idx = oracle.foid(lhs if tensor == 0 else rhs, axis, call.k)
    t_foid = time.perf_counter() - t0

    contract = {"FWD": (1, 1), "DGRAD": (1, 0), "WGRAD": (0, 0)}[op]
    slab = min(K, 2048)
    def cut(x, c):      # the first `slab` contraction positions of a stored operand
        return np.ascontiguousarray(x[:, :slab] if c == oracle.COLS else x[:slab, :])
    t0 = time.perf_counter()
    ac, as_, _ = oracle.iht_quant(cut(lhs, contract[0]), contract[0], 32)
    bc, bs, _ = oracle.iht_quant(cut(rhs, contract[1]), contract[1], 32)
    t_k2 = (time.perf_counter() - t0) * (K / slab)

    # Output tile grown until the product takes a measurable share of the budget.
    side, t_g = 64, 0.0
    while True:
        rows = np.arange(min(side, m)); cols = np.arange(min(side, n))
        t0 = time.perf_counter()
        oracle.gemm_mx(ac, as_, bc, bs, rows, cols)
        t_g = time.perf_counter() - t0
        done = time.perf_counter() - t_all
        if t_g > budget_s / 4 or side >= min(m, n) or done + 4 * t_g > budget_s:
            break
        side *= 2
    t_gemm = t_g * (m * n * K) / (rows.size * cols.size * slab)
    total = t_foid + t_k2 + t_gemm
    return {
        "value": 2.0 * m * n * K / total / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": (f"FOID in full ({t_foid:.2f}s); IHT+quant of both operands on the first "
                   f"{slab} of K={K} contraction positions, x{K / slab:.0f}; fp64 product on a "
                   f"{rows.size}x{cols.size} output tile over that slab, "
                   f"x{m * n * K / (rows.size * cols.size * slab):.3g}; "
                   f"extrapolated call time {total:.1f}s"),
        "sample_wall_s": round(time.perf_counter() - t_all, 2),
    }


def rank_sweep(A, torch, np, wl, call, lhs, rhs, m, n, K, args):
    """Error and latency against the outlier rank (the pages' variant study,
    Fig. 10, on synthetic tensors). Rank 0 is the IHT route with nothing
    extracted; MXFP4 is the plain format without rotation or extraction. The
    error is measured on the fp32 output (before the bf16 rounding) against
    the fp32 product of the same bf16 operands; the latency is that of the
    call with bf16 output."""
    op, T, Din, Dout = call.op, wl.T, wl.Din, wl.Dout
    dev = lhs.device
    base = A.ROUTE_NAME[A.adahop_gemm_plan(op, T, Din, Dout, call.pat_lhs, call.pat_rhs,
                                           call.route, call.k).route]
    if base not in ("OE_LEFT", "OE_RIGHT"):
        sys.exit(f"rank sweep: workload {wl.name} routes to {base}, not an outer OE route")
    torch.backends.cuda.matmul.allow_tf32 = False
    a, b = {"FWD": lambda: (lhs.float(), rhs.float().t().contiguous()),
            "DGRAD": lambda: (lhs.float(), rhs.float()),
            "WGRAD": lambda: (lhs.float().t().contiguous(), rhs.float())}[op]()
    ref = torch.matmul(a, b)
    del a, b
    ref_sq = float((ref.double() ** 2).sum())
    out_shape = {"FWD": (T, Dout), "DGRAD": (T, Din), "WGRAD": (Dout, Din)}[op]
    rows = []
    for name, route, k in ([("MXFP4", "MXFP4", 0), ("IHT", "IHT", 0)] +
                           [(f"{base} k={k}", base, k) for k in (16, 32, 64, 128, 256)]):
        plan = A.adahop_gemm_plan(op, T, Din, Dout, call.pat_lhs, call.pat_rhs, route, max(k, 1))
        ws = torch.empty(max(plan.ws_bytes, 1), dtype=torch.uint8, device=dev)
        o32 = torch.empty(out_shape, dtype=torch.float32, device=dev)
        o16 = torch.empty(out_shape, dtype=torch.bfloat16, device=dev)
        kk = max(k, 1)
        A.adahop_gemm(op, lhs, rhs, call.pat_lhs, call.pat_rhs, route, kk, out=o32, ws=ws)
        torch.cuda.synchronize()
        err = (o32 - ref).double()
        sq = float((err ** 2).sum())
        del err
        for _ in range(args.warmup):
            A.adahop_gemm(op, lhs, rhs, call.pat_lhs, call.pat_rhs, route, kk, out=o16, ws=ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            A.adahop_gemm(op, lhs, rhs, call.pat_lhs, call.pat_rhs, route, kk, out=o16, ws=ws)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / args.steps * 1e3
        rows.append({"variant": name, "route": route, "k": k, "ms": round(ms, 4),
                     "mse": sq / ref.numel(), "rel_frobenius": (sq / ref_sq) ** 0.5})
        print(f"# {name}: {ms:.4f} ms, rel. Frobenius error {(sq / ref_sq) ** 0.5:.4e}",
              file=sys.stderr, flush=True)
        del ws, o32, o16
    print(json.dumps({"rank_sweep": rows, "workload": wl.name, "op": op, "m": m, "n": n, "K": K,
                      "reference": "fp32 product of the bf16 operands (torch.matmul, no TF32)",
                      "error_on": "fp32 output", "latency_on": "bf16 output",
                      "steps": args.steps, "warmup": args.warmup}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed calls first; the clock takes about 20 calls of this size to settle")
    ap.add_argument("--workload", default="l8b_down_wgrad")
    ap.add_argument("--out-dtype", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--route", default=None,
                    choices=["IHT", "OE_LEFT", "OE_RIGHT", "OE_INNER", "MXFP4", "BF16"],
                    help="time the workload's product on this route instead of the one its "
                         "pattern pair selects (BF16: the all-bf16 route)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16-baseline", action="store_true")
    ap.add_argument("--rank-sweep", action="store_true",
                    help="instead of the timed line: for outlier ranks 0 (IHT alone), 16, 32, 64, "
                         "128, 256 and plain MXFP4, print the call's latency and its error against "
                         "an fp32 product of the same bf16 operands")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy 3 times (a known-size reference "
                         "for HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs one product on one GPU; --gpus {args.gpus} is not "
              "supported (the path has no collectives: a data-parallel job runs one call per "
              "GPU on its own shard)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mxfp4_precision_gemms_amd as A

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "copies": 3}))
        return

    wls = workloads()
    if args.workload not in wls:
        sys.exit(f"unknown workload {args.workload}; choose from {sorted(wls)}")
    wl, ci = wls[args.workload]
    call = wl.calls[ci]
    if args.route is not None:
        call = dataclasses.replace(call, route=args.route)
    op = call.op
    T, Din, Dout = wl.T, wl.Din, wl.Dout
    m, n, K = gemm_dims(op, T, Din, Dout)
    dev = torch.device("cuda:0")
    print(f"# workload {wl.name} call {ci}: {op} m={m} n={n} K={K}", file=sys.stderr, flush=True)

    t0 = time.perf_counter()
    lhs_np = wl.tensors[call.lhs].make(0)
    rhs_np = wl.tensors[call.rhs].make(0)
    to_dev = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    lhs, rhs = to_dev(lhs_np), to_dev(rhs_np)
    print(f"# inputs ready in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)

    if args.rank_sweep:
        rank_sweep(A, torch, np, wl, call, lhs, rhs, m, n, K, args)
        return

    out_dtype = torch.bfloat16 if args.out_dtype == "bf16" else torch.float32
    plan = A.adahop_gemm_plan(op, T, Din, Dout, call.pat_lhs, call.pat_rhs, call.route, call.k)
    route = A.ROUTE_NAME[plan.route]
    ws = torch.empty(max(plan.ws_bytes, 1), dtype=torch.uint8, device=dev)
    out_shape = {"FWD": (T, Dout), "DGRAD": (T, Din), "WGRAD": (Dout, Din)}[op]
    out = torch.empty(out_shape, dtype=out_dtype, device=dev)

    def step(events=None):
        A.adahop_gemm(op, lhs, rhs, call.pat_lhs, call.pat_rhs, call.route, call.k,
                      out=out, ws=ws, stage_events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3

    # Stage breakdown and the GEMM's own rate, from a second run of the same
    # steps with HIP events between the stages (each event record adds a few
    # microseconds to the GPU timeline, so the timed steps above record none).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(A.STAGE_EVENTS)]
          for _ in range(args.steps)]
    for e in ev:
        for x in e:
            x.record()
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()

    stage_ms = {}
    for si, name in enumerate(A.STAGES):
        stage_ms[name] = float(np.mean([e[si].elapsed_time(e[si + 1]) for e in ev]))
    call_ms = float(np.mean([e[0].elapsed_time(e[-1]) for e in ev]))
    flops = 2.0 * m * n * K
    value = flops / (ms_per_step / 1e3) / 1e12
    gemm_ms = stage_ms["gemm"]
    achieved = flops / (gemm_ms / 1e3) / 1e12
    bf16 = route == "BF16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP4_TFLOPS

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "mxfp4",
        "data": "synthetic",
        "config": {"workload": wl.name, "op": op, "route": route, "m": m, "n": n, "K": K,
                   "oe_rank": plan.k, "pattern_pair": call.pat_lhs + call.pat_rhs,
                   "out_dtype": args.out_dtype},
        "pct_mxfp4_peak": round(100 * value / PEAK_FP4_TFLOPS, 2),
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stages_note": ("quant_lhs and quant_rhs are the K-major copies of operands stored "
                        "across K that cannot be read in place (empty when there are none); gemm "
                        "is the bf16 MFMA kernel plus, when its last round is split along K, the "
                        "fixup kernel") if bf16 else
                       ("the operand FOID does not scan is quantized on a second stream, beside "
                        "FOID, the other quantization and the outlier product: its slot is empty "
                        "and the other slots overlap it; gemm is the MFMA kernel plus, when its "
                        "last round is split along K, the fixup kernel")
                       if route in ("OE_LEFT", "OE_RIGHT") else
                       ("gemm is the MFMA kernel plus, when its last round is split along K, "
                        "the fixup kernel"),
        "call_ms_events": round(call_ms, 4),
        "roofline": {"bound": "mfma",
                     "kernel": ("gemm_mx_ring8_kernel<bf16> + gemm_split_fixup_kernel (bf16 MFMA "
                                "GEMM; the fixup adds the K-parts of a split last round)") if bf16 else
                               ("gemm_mx_ring8_kernel + gemm_split_fixup_kernel (FP4 MFMA GEMM, "
                                "fused scatter-add epilogue; the fixup adds the K-parts of a "
                                "split last round)"),
                     "achieved": round(achieved, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": None},
    }
    if bf16:
        del result["pct_mxfp4_peak"]
    traffic, note = measured_traffic(wl.name, TRAFFIC_SUMMARY_BF16 if bf16 else TRAFFIC_SUMMARY)
    result["roofline"]["traffic"] = None if traffic is None else round(traffic)
    result["roofline"]["traffic_note"] = note

    if not args.no_bf16_baseline:
        # All-bf16 reference product on hipBLASLt (torch.matmul, 2-D), same
        # shapes, in the faster of two operand arrangements: the stored
        # tensors as (transposed) views, or the transposed operand made
        # contiguous beforehand (its copy not timed).
        arrangements = {
            "FWD": (("X, W^T view", lambda: (lhs, rhs.t())),
                    ("X, W^T contiguous", lambda: (lhs, rhs.t().contiguous()))),
            "DGRAD": (("GY, W", lambda: (lhs, rhs)),
                      ("GY, W column-major", lambda: (lhs, rhs.t().contiguous().t()))),
            "WGRAD": (("GY^T view, X", lambda: (lhs.t(), rhs)),
                      ("GY^T contiguous, X", lambda: (lhs.t().contiguous(), rhs))),
        }[op]
        best = None
        for name, make in arrangements:
            a2 = make()
            for _ in range(3):
                torch.matmul(*a2)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(max(3, args.steps // 2)):
                torch.matmul(*a2)
            torch.cuda.synchronize()
            bms = (time.perf_counter() - t0) / max(3, args.steps // 2) * 1e3
            del a2
            if best is None or bms < best[1]:
                best = (name, bms)
        result["bf16_matmul_ms"] = round(best[1], 4)
        result["bf16_matmul_operands"] = best[0]
        result["speedup_vs_bf16_matmul"] = round(best[1] / ms_per_step, 3)
        # hipBLASLt's own MXFP4 GEMM (torch._scaled_mm on packed E2M1 codes
        # with unit E8M0 scales), same m, n, K: a library reference for the
        # GEMM stage alone.
        try:
            if bf16:
                raise NotImplementedError("the BF16 route has no MXFP4 GEMM stage")
            f4 = torch.float4_e2m1fn_x2
            e8 = torch.float8_e8m0fnu
            qa = torch.randint(0, 256, (m, K // 2), dtype=torch.uint8, device=dev).view(f4)
            qb = torch.randint(0, 256, (n, K // 2), dtype=torch.uint8, device=dev).view(f4)
            sa = torch.full((m, K // 32), 127, dtype=torch.uint8, device=dev).view(e8)
            sb = torch.full((n, K // 32), 127, dtype=torch.uint8, device=dev).view(e8)
            mm = lambda: torch._scaled_mm(qa, qb.t(), sa, sb, out_dtype=torch.bfloat16)
            for _ in range(3):
                mm()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(max(3, args.steps // 2)):
                mm()
            torch.cuda.synchronize()
            fms = (time.perf_counter() - t0) / max(3, args.steps // 2) * 1e3
            result["hipblaslt_mxfp4_gemm_ms"] = round(fms, 4)
            result["gemm_stage_speedup_vs_hipblaslt_mxfp4"] = round(fms / gemm_ms, 3)
            del qa, qb, sa, sb
        except Exception as ex:          # no MXFP4 GEMM in this torch build
            result["hipblaslt_mxfp4_gemm_ms"] = None
            if not bf16:
                print(f"# hipBLASLt MXFP4 reference unavailable: {type(ex).__name__}",
                      file=sys.stderr)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(op, lhs_np, rhs_np, T, Din, Dout, call, m, n, K)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
