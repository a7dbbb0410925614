"""GPU line scores (FOID's score of every row or column) bit-exact against
the oracle, and the calibration of every synthetic workload tensor at full
size: the pattern planted in it, the same as the oracle's classification."""
import numpy as np
import pytest
import torch

import mxfp4_precision_gemms_amd as A
import oracle
from synth import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def dev_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)


SCORE_CASES = [
    # rows, cols, axis, probe, pattern
    (300, 520, "ROWS", 64, "R"), (300, 520, "COLS", 64, "C"),
    (300, 520, "COLS", 17, "C"), (300, 520, "ROWS", 1000, "N"),    # probe beyond the line
    (1, 64, "ROWS", 64, "N"), (64, 1, "COLS", 64, "N"),
    (2049, 77, "ROWS", 64, "R"), (77, 2049, "COLS", 300, "C"),
]


@pytest.mark.parametrize("case", SCORE_CASES, ids=[str(c) for c in SCORE_CASES])
def test_line_scores_bit_exact(case):
    rows, cols, axis, probe, pat = case
    say("line scores", case)
    dim = rows if pat == "R" else cols
    spec = W.TensorSpec("X", rows, cols, pat, 0 if pat == "N" else max(1, dim // 50), 40.0)
    t = spec.make(rows + cols)
    got = A.adahop_line_scores(dev_bf16(t), axis, probe).cpu().numpy()
    ref = oracle.line_scores(t, oracle.ROWS if axis == "ROWS" else oracle.COLS, probe)
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))


def test_line_scores_strided_rows():
    # a view with ld > cols: the first 200 columns of a [128, 264] tensor
    t = W.TensorSpec("W", 128, 264, "C", 4, 30.0).make(9)
    d = dev_bf16(t)[:, :200]
    assert d.stride(0) == 264
    for axis in ("ROWS", "COLS"):
        got = A.adahop_line_scores(d, axis, 64).cpu().numpy()
        ref = oracle.line_scores(np.ascontiguousarray(t[:, :200]),
                                 oracle.ROWS if axis == "ROWS" else oracle.COLS, 64)
        assert np.array_equal(got.view(np.uint64), ref.view(np.uint64)), axis


def workload_tensors():
    seen = {}
    for wl in (W.tiny_fwd(), W.l32_1b_up_fwd(), W.l31_8b_down_wgrad(),
               W.l31_8b_gateup_fwd_dgrad(), W.l31_8b_oproj_triplet(8)):
        for name, spec in wl.tensors.items():
            key = (spec.rows, spec.cols, name, spec.pattern, spec.n_lines, spec.factor)
            seen.setdefault(key, (wl.name, spec))
    return list(seen.values())


TENSORS = workload_tensors()


@pytest.mark.parametrize("wl_spec", TENSORS,
                         ids=[f"{w}-{s.name}-{s.rows}x{s.cols}" for w, s in TENSORS])
def test_calibrate_workload_tensor(wl_spec):
    wl_name, spec = wl_spec
    say("calibrate", wl_name, spec.name, (spec.rows, spec.cols), spec.pattern)
    t = spec.make(0)
    d = dev_bf16(t)
    rs = A.adahop_line_scores(d, "ROWS", 64)
    cs = A.adahop_line_scores(d, "COLS", 64)
    got = A.adahop_classify_pattern(rs, cs)
    ref_rs = oracle.line_scores(t, oracle.ROWS, 64)
    ref_cs = oracle.line_scores(t, oracle.COLS, 64)
    assert np.array_equal(rs.cpu().numpy().view(np.uint64), ref_rs.view(np.uint64))
    assert np.array_equal(cs.cpu().numpy().view(np.uint64), ref_cs.view(np.uint64))
    assert got == oracle.classify_pattern(ref_rs, ref_cs, A.CLASSIFY_THRESHOLD) == spec.pattern
