"""Whole adahop_gemm calls captured into a HIP graph (torch.cuda.graph) and
replayed: every replay must equal the eager call bit for bit (the path is
deterministic). Covers FOID's selection sharing its launch with the other
operand's quantization, the second-stream fork and join under capture
(taken when that launch does not apply and the two operands exceed 96 MB of
bf16), the FOID counter reset inside the graph and the K-split of the GEMM's
last round. Between replays the program does its own
eager work (clearing the output) and synchronizes."""
import numpy as np
import pytest
import torch

import mxfp4_precision_gemms_amd as A
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def operands(op, T, Din, Dout, pl, pr, seed):
    shapes = {"FWD": ((T, Din), (Dout, Din)), "DGRAD": ((T, Dout), (Dout, Din)),
              "WGRAD": ((T, Dout), (T, Din))}[op]
    out = []
    for t, (pat, shape) in enumerate(zip((pl, pr), shapes)):
        axis = {"R": 0, "C": 1, "N": -1}[pat]
        dim = shape[0] if pat == "R" else shape[1]
        lines = synth.pick_lines(seed, 50 + t, dim, max(1, dim // 100)) if pat != "N" else None
        out.append(synth.fill_bf16(shape[0], shape[1], seed, 60 + t, 0.02, axis, lines, 50.0))
    return [torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
            for x in out]


CASES = [
    # op, T, Din, Dout, pattern pair, route (None: by the pattern pair)
    ("WGRAD", 4096, 768, 512, "R", "C", "OE_RIGHT"),   # one stream; K = 4096: split last round
    ("FWD", 1024, 1024, 520, "R", "N", "OE_LEFT"),     # one stream, FOID over 1024 rows
    # operands above 96 MB together: FOID's selection shares its launch with
    # the other operand's quantization (down the columns)
    ("WGRAD", 8192, 6400, 256, "R", "C", "OE_RIGHT"),  # X [8192, 6400] scanned by columns
    ("DGRAD", 16384, 256, 3072, "R", "N", "OE_LEFT"),  # GY [16384, 3072] scanned by rows
    # above 96 MB, W quantized along its rows in FOID's launch
    ("FWD", 16384, 3072, 256, "R", "N", "OE_LEFT"),    # X [16384, 3072] scanned by rows
    # above 96 MB with FOID over 70016 rows (three selection levels): the
    # second stream's fork and join
    ("FWD", 70016, 768, 256, "R", "N", "OE_LEFT"),
    ("FWD", 512, 2048, 384, "C", "N", "OE_INNER"),     # asked for: both operands zeroed, one stream
    ("WGRAD", 2048, 320, 300, "C", "C", "BF16"),       # X in place, GY copied; 4 tiles in 4 K-parts
]


@pytest.mark.parametrize("case", CASES, ids=[c[-1] for c in CASES])
def test_graph_replay_matches_eager(case):
    op, T, Din, Dout, pl, pr, route = case
    lhs, rhs = operands(op, T, Din, Dout, pl, pr, seed=T + Dout)
    ask = route if route == "OE_INNER" else None
    plan = A.adahop_gemm_plan(op, T, Din, Dout, pl, pr, ask, 16)
    assert A.ROUTE_NAME[plan.route] == route
    say("graph", case)
    eager = A.adahop_gemm(op, lhs, rhs, pl, pr, ask, 16)
    torch.cuda.synchronize()

    ws = torch.empty(max(plan.ws_bytes, 1), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):            # warm-up off the capture, as torch advises
        A.adahop_gemm(op, lhs, rhs, pl, pr, ask, 16, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        A.adahop_gemm(op, lhs, rhs, pl, pr, ask, 16, out=out, ws=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
    # and an eager call after the replays still agrees
    again = A.adahop_gemm(op, lhs, rhs, pl, pr, ask, 16)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), eager.view(torch.int16))
