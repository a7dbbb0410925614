"""Calls on different streams and from different host threads: the
library's per-device second stream is shared under a lock, each call's
fork and join stay ordered on its own stream, and every result equals the
same call run alone."""
import threading

import numpy as np
import pytest
import torch

import mxfp4_precision_gemms_amd as A
from test_gpu_parity import operands

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # op, T, Din, Dout, pl, pr, k  (OE_RIGHT / OE_LEFT with the operands above
    # 96 MB together: FOID's launch quantizes the other operand too, down its
    # columns or along its rows; with k above 256 it cannot, and the second
    # stream is used)
    ("WGRAD", 8192, 6400, 256, "R", "C", 16),
    ("DGRAD", 16384, 256, 3072, "R", "N", 8),
    ("FWD", 16384, 3072, 256, "R", "N", 8),
    ("FWD", 16384, 3072, 256, "R", "N", 300),
    ("WGRAD", 1024, 384, 512, "R", "C", 16),
    ("DGRAD", 512, 640, 1024, "R", "N", 8),
    ("WGRAD", 2048, 256, 200, "C", "N", 32),
    ("FWD", 300, 1024, 200, "R", "N", 8),
    ("WGRAD", 2048, 320, 300, "C", "C", 8),     # BF16: X in place, GY copied, split tiles
]


def dev_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)


def inputs():
    out = []
    for i, (op, T, Din, Dout, pl, pr, k) in enumerate(CASES):
        lhs, rhs = operands(op, T, Din, Dout, pl, pr, seed=77 + i)
        out.append((op, dev_bf16(lhs), dev_bf16(rhs), pl, pr, k))
    return out


def call(c, stream=None):
    op, L, R, pl, pr, k = c
    with torch.cuda.stream(stream or torch.cuda.current_stream()):
        return A.adahop_gemm(op, L, R, pl, pr, None, k)


def test_concurrent_streams_match_serial():
    data = inputs()
    ref = [call(c) for c in data]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in data]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        got = [call(c, s) for c, s in zip(data, streams)]
        for s in streams:
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for r, g in zip(ref, got):
            assert torch.equal(r.view(torch.int16), g.view(torch.int16))


def test_host_threads_match_serial():
    data = inputs()
    ref = [call(c) for c in data]
    torch.cuda.synchronize()
    results = [None] * len(data)
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            outs = []
            for _ in range(4):
                outs.append(call(data[i], s))
            s.synchronize()
            results[i] = outs
        except Exception as e:   # reported below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(data))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for r, outs in zip(ref, results):
        for g in outs:
            assert torch.equal(r.view(torch.int16), g.view(torch.int16))
