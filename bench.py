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
`--sweep-oproj` prints one line per batch size 1..16 and product of the
Llama3.1-8B o_proj triplet (Fig. 6 per batch size, Table 3's rows): the
AdaHOP route, plain MXFP4, this library's BF16 route and hipBLASLt's bf16
GEMM. `--from-context` times a weight gradient from the saved forward
context of X (adahop_gemm_wgrad_ctx) instead of from X.

Timing: W untimed warm-up calls (preceded by untimed calls for --settle-ms
of wall time so that the clock has settled, reported as settle_calls), then
K calls back to back timed by the host clock around a device
synchronization (value, ms_per_step); per-call HIP events on the call's
stream give the median and p10/p90 of the same calls back to back, and
again with a 512 MB buffer written between calls (outside each call's
events) so that no operand is left in the L2 or the 256 MB Infinity
Cache.
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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def quantiles(ms):
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4)}


def settle(torch, step, settle_ms):
    """Untimed calls until settle_ms of wall time has passed (the shader clock
    takes a few tens of calls of a millisecond to reach its steady state)."""
    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def per_call_ms(torch, step, steps, flush=None):
    """Per-call times from HIP events on the current stream (the library
    enqueues every launch of a call there, its second stream joined back)."""
    ev = []
    for _ in range(steps):
        if flush is not None:
            flush()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


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
        "cpu_model": cpu_model(),
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


def mfma_ceiling(torch, np, args):
    """The FP4 matrix cores' steady-state rate and shader clock with no memory
    traffic (libadahop_probe.so): one workgroup per CU, 8 independent scaled
    32x32x64 FP4 MFMAs per wave on switching register operands, launches of
    about 0.1 s back to back. The practical ceiling under the device's power
    limit for any FP4 kernel, against the nominal 10.1 PFLOP/s (2.4 GHz)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "mxfp4_precision_gemms_amd", "libadahop_probe.so"))
    for fn in (lib.adahop_probe_mfma_fp4, lib.adahop_probe_mfma_fp4_16, lib.adahop_probe_lds_read):
        fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                       ctypes.c_void_p]
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    iters, launches = 400000, 5
    scratch = torch.empty(blocks * 16 + 2048, dtype=torch.uint8, device="cuda:0")
    cyc = np.zeros(launches)
    tick = np.zeros(launches)
    rc = lib.adahop_probe_mfma_fp4(blocks, iters, launches, scratch.data_ptr(), cyc.ctypes.data,
                                   tick.ctypes.data)
    if rc != 0:
        sys.exit(f"mfma probe failed: hipError {rc}")
    mfmas_per_wave = 8 * iters
    clock = cyc / tick * 0.1                              # GHz (ticks at 100 MHz)
    util = mfmas_per_wave * 2 * 32 / cyc                  # 2 waves per SIMD, 32 cycles per MFMA
    tflops = blocks * 8 * mfmas_per_wave * 131072 / (tick / 1e8) / 1e12
    # The same multiply-adds as 16x16x128 MFMAs (half the accumulator traffic per MAC).
    cyc16 = np.zeros(launches)
    tick16 = np.zeros(launches)
    rc = lib.adahop_probe_mfma_fp4_16(blocks, iters, launches, scratch.data_ptr(), cyc16.ctypes.data,
                                      tick16.ctypes.data)
    if rc != 0:
        sys.exit(f"mfma probe (16x16x128) failed: hipError {rc}")
    clock16 = cyc16 / tick16 * 0.1
    util16 = mfmas_per_wave * 2 * 32 / cyc16          # 16 MFMAs of 16 cycles per iteration
    tflops16 = blocks * 8 * mfmas_per_wave * 131072 / (tick16 / 1e8) / 1e12
    # One wave per SIMD, 64 16x16x128 blocks per wave (128 x 128 outputs): with
    # the fragments in registers, and read from LDS as a GEMM would.
    lib.adahop_probe_mfma_fp4_16_w1.argtypes = [ctypes.c_int] + [ctypes.c_int, ctypes.c_int,
                                                                 ctypes.c_int, ctypes.c_void_p,
                                                                 ctypes.c_void_p, ctypes.c_void_p]
    w1 = {}
    w1_iters = 150000
    for lds in (0, 1):
        c1, t1 = np.zeros(launches), np.zeros(launches)
        rc = lib.adahop_probe_mfma_fp4_16_w1(lds, blocks, w1_iters, launches, scratch.data_ptr(),
                                             c1.ctypes.data, t1.ctypes.data)
        if rc != 0:
            sys.exit(f"mfma probe (one wave per SIMD) failed: hipError {rc}")
        tf = blocks * 4 * 64 * w1_iters * 65536 / (t1 / 1e8) / 1e12
        w1["lds" if lds else "registers"] = {
            "launch_ms": [round(float(t) / 1e5, 2) for t in t1],
            "clock_ghz": [round(float(c), 3) for c in c1 / t1 * 0.1],
            "mfma_busy": [round(float(u), 4) for u in w1_iters * 64 * 16 / c1],
            "tflops": [round(float(t), 1) for t in tf],
            "frac_of_nominal_peak": [round(float(t) / PEAK_FP4_TFLOPS, 4) for t in tf]}
    lit = 20000
    lc, lt = np.zeros(3), np.zeros(3)
    rc = lib.adahop_probe_lds_read(blocks, lit, 3, scratch.data_ptr(), lc.ctypes.data, lt.ctypes.data)
    if rc != 0:
        sys.exit(f"lds probe failed: hipError {rc}")
    lds_bpc = 8 * 512 * 16 * lit / lc                   # bytes per shader clock per CU
    print(json.dumps({"lds_read": {"bytes_per_clk_per_cu": [round(float(b), 1) for b in lds_bpc],
                                   "clock_ghz": [round(float(c), 3) for c in lc / lt * 0.1]},
                      "mfma_ceiling": {
        "kernel": "8 x v_mfma_scale_f32_32x32x64_f8f6f4 (E2M1 x E2M1) per wave per iteration, "
                  "register operands, 8 waves per CU",
        "cus": blocks, "launch_ms": [round(float(t) / 1e5, 2) for t in tick],
        "clock_ghz": [round(float(c), 3) for c in clock],
        "mfma_busy": [round(float(u), 4) for u in util],
        "tflops": [round(float(t), 1) for t in tflops],
        "frac_of_nominal_peak": [round(float(t) / PEAK_FP4_TFLOPS, 4) for t in tflops]},
                      "mfma_ceiling_16x16x128": {
        "kernel": "16 x v_mfma_scale_f32_16x16x128_f8f6f4 (E2M1 x E2M1) per wave per iteration "
                  "(the same multiply-adds), register operands, 8 waves per CU",
        "launch_ms": [round(float(t) / 1e5, 2) for t in tick16],
        "clock_ghz": [round(float(c), 3) for c in clock16],
        "mfma_busy": [round(float(u), 4) for u in util16],
        "tflops": [round(float(t), 1) for t in tflops16],
        "frac_of_nominal_peak": [round(float(t) / PEAK_FP4_TFLOPS, 4) for t in tflops16]},
                      "mfma_16x16x128_one_wave_per_simd": dict(
        kernel="64 x v_mfma_scale_f32_16x16x128_f8f6f4 per wave per iteration, 4 waves per CU "
               "(accumulators in AGPRs); 'lds': the next iteration's 16 fragments read from LDS "
               "during the MFMAs", **w1)}), flush=True)


def hbm_ceiling(torch, np, args):
    """HBM streaming rates (libadahop_probe.so) on two 2 GiB buffers: reads
    with ordinary and non-temporal loads, writes, copies, and the read pattern
    of the column-direction quantizer; median and best of 12 launches."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "mxfp4_precision_gemms_amd", "libadahop_probe.so"))
    fn = lib.adahop_probe_hbm
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    nbytes = 2 << 30
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(2)
    sink = torch.empty(1024, dtype=torch.uint8, device="cuda:0")
    grid = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    launches = 12
    out = {}
    for name, mode, nt, moved in (("read", 0, 0, nbytes), ("read_nt", 0, 1, nbytes),
                                  ("write", 1, 0, nbytes), ("copy", 2, 0, 2 * nbytes),
                                  ("copy_nt_loads", 2, 1, 2 * nbytes),
                                  ("quantizer_column_blocks_read", 3, 0, (nbytes // 28672) // 128 * 128 * 28672),
                                  ("quantizer_column_blocks_read_nt", 3, 1, (nbytes // 28672) // 128 * 128 * 28672)):
        ms = np.zeros(launches, dtype=np.float32)
        rc = fn(mode, nt, a.data_ptr(), b.data_ptr(), nbytes, grid, launches, sink.data_ptr(),
                ms.ctypes.data)
        if rc != 0:
            sys.exit(f"hbm probe failed: hipError {rc}")
        t = np.sort(ms[2:])                                 # the first two launches warm up
        out[name] = {"tb_per_s_median": round(moved / float(np.median(t)) / 1e9, 2),
                     "tb_per_s_best": round(moved / float(t[0]) / 1e9, 2),
                     "bytes_moved": int(moved)}
    print(json.dumps({"hbm_stream": out, "grid": grid, "launches": launches,
                      "nominal_tb_per_s": 8.0}), flush=True)


def sweep_oproj(A, torch, np, args):
    """One JSON line per (batch size, product) of the Llama3.1-8B o_proj
    triplet: effective TFLOP/s of the AdaHOP route with its GEMM stage's
    roofline fraction, beside plain MXFP4 (no rotation, no extraction), this
    library's BF16 route and hipBLASLt's bf16 GEMM (2-D torch.matmul, the
    faster of two operand arrangements), all on the same synthetic tensors,
    per-call medians over back-to-back calls."""
    from synth import workloads as W
    dev = torch.device("cuda:0")
    to_dev = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    for bs in (1, 2, 4, 8, 16):
        wl = W.l31_8b_oproj_triplet(bs)
        T, Din, Dout = wl.T, wl.Din, wl.Dout
        tens = {k: to_dev(v.make(0)) for k, v in wl.tensors.items()}
        for call in wl.calls:
            op = call.op
            m, n, K = gemm_dims(op, T, Din, Dout)
            flops = 2.0 * m * n * K
            lhs, rhs = tens[call.lhs], tens[call.rhs]
            out_shape = {"FWD": (T, Dout), "DGRAD": (T, Din), "WGRAD": (Dout, Din)}[op]
            out = torch.empty(out_shape, dtype=torch.bfloat16, device=dev)
            line = {"sweep": "llama3.1-8b_oproj", "bs": bs, "op": op, "m": m, "n": n, "K": K,
                    "pattern_pair": call.pat_lhs + call.pat_rhs}
            for label, route in (("adahop", call.route), ("mxfp4", "MXFP4"), ("bf16_route", "BF16")):
                plan = A.adahop_gemm_plan(op, T, Din, Dout, call.pat_lhs, call.pat_rhs, route, call.k)
                ws = torch.empty(max(plan.ws_bytes, 1), dtype=torch.uint8, device=dev)
                step = lambda ev=None: A.adahop_gemm(op, lhs, rhs, call.pat_lhs, call.pat_rhs, route,
                                                     call.k, out=out, ws=ws, stage_events=ev)
                settle(torch, step, args.settle_ms / 4)
                for _ in range(args.warmup):
                    step()
                ms = float(np.median(per_call_ms(torch, step, args.steps)))
                entry = {"route": A.ROUTE_NAME[plan.route], "ms": round(ms, 4),
                         "tflops": round(flops / ms / 1e9, 1)}
                if label == "adahop":
                    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(A.STAGE_EVENTS)]
                           for _ in range(args.steps)]
                    for e in evs:
                        step(e)
                    torch.cuda.synchronize()
                    gms = float(np.median([e[4].elapsed_time(e[6]) for e in evs]))
                    kms = float(np.median([e[4].elapsed_time(e[5]) for e in evs]))
                    entry["gemm_stage_ms"] = round(gms, 4)
                    entry["gemm_frac_mxfp4_peak"] = round(flops / gms / 1e9 / PEAK_FP4_TFLOPS, 4)
                    entry["gemm_kernel_ms"] = round(kms, 4)
                    entry["gemm_kernel_frac_mxfp4_peak"] = round(flops / kms / 1e9 / PEAK_FP4_TFLOPS, 4)
                    entry["pct_mxfp4_peak"] = round(100 * flops / ms / 1e9 / PEAK_FP4_TFLOPS, 2)
                line[label] = entry
                del ws
            if op == "WGRAD":
                cplan = A.adahop_ctx_plan(T, Din, Dout, call.pat_lhs, call.pat_rhs, call.route, call.k)
                ctx = A.adahop_ctx_save(rhs, Dout, call.pat_lhs, call.pat_rhs, call.route, call.k)
                ws = torch.empty(max(cplan.wgrad_ws_bytes, 1), dtype=torch.uint8, device=dev)
                step = lambda: A.adahop_gemm_wgrad_ctx(lhs, ctx, Din, call.pat_lhs, call.pat_rhs,
                                                       call.route, call.k, out=out, ws=ws)
                for _ in range(args.warmup):
                    step()
                ms = float(np.median(per_call_ms(torch, step, args.steps)))
                save = lambda: A.adahop_ctx_save(rhs, Dout, call.pat_lhs, call.pat_rhs, call.route,
                                                 call.k, ctx=ctx)
                for _ in range(3):
                    save()
                sms = float(np.median(per_call_ms(torch, save, args.steps)))
                line["adahop_from_context"] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
                                               "ctx_save_ms": round(sms, 4),
                                               "ctx_mib": round(cplan.ctx_bytes / 2 ** 20, 1),
                                               "x_bf16_mib": round(2 * T * Din / 2 ** 20, 1)}
                del ctx, ws
            arr = {"FWD": ((lambda: (lhs, rhs.t())), (lambda: (lhs, rhs.t().contiguous()))),
                   "DGRAD": ((lambda: (lhs, rhs)), (lambda: (lhs, rhs.t().contiguous().t()))),
                   "WGRAD": ((lambda: (lhs.t(), rhs)), (lambda: (lhs.t().contiguous(), rhs)))}[op]
            best = None
            for mk in arr:
                a2 = mk()
                for _ in range(3):
                    torch.matmul(*a2)
                ms = float(np.median(per_call_ms(torch, lambda: torch.matmul(*a2), args.steps)))
                best = ms if best is None else min(best, ms)
                del a2
            line["hipblaslt_bf16"] = {"ms": round(best, 4), "tflops": round(flops / best / 1e9, 1)}
            line["speedup_vs_hipblaslt_bf16"] = round(best / line["adahop"]["ms"], 3)
            line["speedup_vs_bf16_route"] = round(line["bf16_route"]["ms"] / line["adahop"]["ms"], 3)
            line["adahop_vs_mxfp4"] = round(line["mxfp4"]["ms"] / line["adahop"]["ms"], 3)
            print(json.dumps(line), flush=True)
        del tens


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
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed calls for this much wall time before the warm-up calls, so that "
                         "the shader clock has reached its steady state (0: none)")
    ap.add_argument("--no-flush-timing", action="store_true",
                    help="skip the per-call timing with the caches flushed between calls")
    ap.add_argument("--sweep-oproj", action="store_true",
                    help="instead of the timed line: the o_proj triplet at batch sizes 1-16 against "
                         "plain MXFP4, the BF16 route and hipBLASLt bf16, one JSON line each")
    ap.add_argument("--oe-in-quant", action="store_true",
                    help="OE_LEFT / OE_RIGHT: form the outlier product in the quantization of the "
                         "operand FOID does not scan (one read of it; adahop_gemm_ex) instead of "
                         "inside the GEMM launch")
    ap.add_argument("--from-context", action="store_true",
                    help="time a weight gradient from the saved forward context of X "
                         "(adahop_gemm_wgrad_ctx) instead of from X")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="instead of the timed line: the FP4 matrix cores' rate and clock with no "
                         "memory traffic (the practical ceiling under the power limit)")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="HBM streaming rates of read, write and copy probes, and of the "
                         "column quantizer's read pattern")
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

    if args.sweep_oproj:
        sweep_oproj(A, torch, np, args)
        return
    if args.mfma_ceiling:
        mfma_ceiling(torch, np, args)
        return
    if args.hbm_ceiling:
        hbm_ceiling(torch, np, args)
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
    plan = A.adahop_gemm_plan(op, T, Din, Dout, call.pat_lhs, call.pat_rhs, call.route, call.k,
                              args.oe_in_quant)
    route = A.ROUTE_NAME[plan.route]
    if args.oe_in_quant and (args.from_context or not plan.oe_in_quant):
        sys.exit("--oe-in-quant applies to OE_LEFT / OE_RIGHT calls whose other operand is "
                 "quantized down its columns, with k <= 64, not from a context")
    out_shape = {"FWD": (T, Dout), "DGRAD": (T, Din), "WGRAD": (Dout, Din)}[op]
    out = torch.empty(out_shape, dtype=out_dtype, device=dev)
    ctx_info = None
    if args.from_context:
        if op != "WGRAD":
            sys.exit("--from-context applies to weight-gradient workloads")
        cplan = A.adahop_ctx_plan(T, Din, Dout, call.pat_lhs, call.pat_rhs, call.route, call.k)
        ctx = A.adahop_ctx_save(rhs, Dout, call.pat_lhs, call.pat_rhs, call.route, call.k)
        ws = torch.empty(max(cplan.wgrad_ws_bytes, 1), dtype=torch.uint8, device=dev)
        save = lambda: A.adahop_ctx_save(rhs, Dout, call.pat_lhs, call.pat_rhs, call.route, call.k,
                                         ctx=ctx)
        for _ in range(3):
            save()
        ctx_info = {"ctx_save_ms": quantiles(per_call_ms(torch, save, args.steps)),
                    "ctx_bytes": cplan.ctx_bytes, "x_bf16_bytes": 2 * T * Din}

        def step(events=None):
            A.adahop_gemm_wgrad_ctx(lhs, ctx, Din, call.pat_lhs, call.pat_rhs, call.route, call.k,
                                    out=out, ws=ws, stage_events=events)
    else:
        ws = torch.empty(max(plan.ws_bytes, 1), dtype=torch.uint8, device=dev)

        def step(events=None):
            A.adahop_gemm(op, lhs, rhs, call.pat_lhs, call.pat_rhs, call.route, call.k,
                          out=out, ws=ws, stage_events=events, oe_in_quant=args.oe_in_quant)

    settle_calls = settle(torch, step, args.settle_ms) if args.settle_ms > 0 else 0
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3

    # The same number of calls again, each between HIP events: back to back,
    # then with the caches flushed before every call (outside its events).
    per_call = quantiles(per_call_ms(torch, step, args.steps))
    per_call_flushed = None
    if not args.no_flush_timing:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        flush = lambda: scratch.fill_(1)
        per_call_flushed = quantiles(per_call_ms(torch, step, args.steps, flush))
        del scratch

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
    # The GEMM's main kernel alone (events 4 -> 5) and the whole GEMM stage
    # with the kernels that finish its output (4 -> 6): medians over the steps.
    gemm_ms = float(np.median([e[4].elapsed_time(e[5]) for e in ev]))
    gemm_stage_ms = float(np.median([e[4].elapsed_time(e[6]) for e in ev]))
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
        "settle_calls": settle_calls,
        "ms_per_step": round(ms_per_step, 4),
        "per_call_ms": per_call,
        "per_call_ms_cache_flushed": per_call_flushed,
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
                        "is the bf16 MFMA kernel, gemm_tail the fixup kernel of a split last "
                        "round") if bf16 else
                       ("one read of the operand FOID does not scan: FOID, the scanned operand's "
                        "quantization (which gathers the lines), the other's forming the outlier "
                        "product's partial sums (with OE_RIGHT in the oe_product slot, the lhs "
                        "slot empty), their sum in order (oe_product), the GEMM (its epilogue "
                        "adds the sum to the extracted lines), gemm_tail the fixup kernel of a "
                        "split last round")
                       if args.oe_in_quant else
                       ("the operand FOID does not scan is quantized beside FOID: in FOID's own "
                        "launch (the foid slot holds both, that operand's slot is empty) when "
                        "the selection takes at most two levels, else on a second stream when "
                        "the operands exceed 96 MB (its "
                        "slot empty, the other slots overlap it), else after FOID; when the wide "
                        "outlier factor is stored across K and k <= 64 the outlier product runs "
                        "as work items of the GEMM kernel (its own slot empty), else before it; "
                        "gemm is the MFMA kernel, gemm_tail the fixup kernel of a split last "
                        "round and the kernel that adds the outlier product to the extracted "
                        "lines")
                       if route in ("OE_LEFT", "OE_RIGHT") else
                       ("gemm is the MFMA kernel, gemm_tail the fixup kernel of a split last "
                        "round"),
        "call_ms_events": round(call_ms, 4),
        "gemm_kernel_ms_median": round(gemm_ms, 4),
        "gemm_stage_ms_median": round(gemm_stage_ms, 4),
        "gemm_stage_frac": round(flops / (gemm_stage_ms / 1e3) / 1e12 / peak, 4),
        "roofline": {"bound": "mfma",
                     "kernel": ("gemm_mx_ring8_kernel<false, true, TA, TB> (bf16 MFMA GEMM, main "
                                "kernel alone)") if bf16 else
                               ("gemm_mx_ring8_kernel<true, false, false, false> (FP4 MFMA GEMM, "
                                "main kernel alone; its first workgroups also compute the rank-k "
                                "bf16 outlier product as work items, whose 2mkK flops are not "
                                "counted)") if route in ("OE_LEFT", "OE_RIGHT") and not args.oe_in_quant
                               else
                               ("gemm_mx_ring8_kernel<true, false, false, false> (FP4 MFMA GEMM, "
                                "main kernel alone)"),
                     "achieved": round(achieved, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": None},
    }
    if bf16:
        del result["pct_mxfp4_peak"]
    if ctx_info is not None:
        result["config"]["from_context"] = True
        result["context"] = ctx_info
        result["stages_note"] = ("weight gradient from the saved forward context of X: FOID and X's "
                                 "quantization ran in the forward (context save, timed apart in "
                                 "context.ctx_save_ms); quant_lhs is GY's")
    traffic, note = measured_traffic(wl.name, TRAFFIC_SUMMARY_BF16 if bf16 else TRAFFIC_SUMMARY)
    if args.oe_in_quant:
        result["config"]["oe_in_quant"] = True
        traffic, note = None, "the counters were taken on the default path (outlier items in the GEMM)"
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
            result["gemm_stage_speedup_vs_hipblaslt_mxfp4"] = round(fms / gemm_stage_ms, 3)
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
