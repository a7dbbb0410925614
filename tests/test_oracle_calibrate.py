"""Pins of the oracle's pattern calibration (line scores + classification).

The pages name the three patterns (Table 1) and show them (Fig. 4, Fig. 8)
but give no numeric test; the rule is this repository's reading, stated in
oracle.classify_pattern. Pinned here: a hand-computed case whose ratios are
exact, invariances the rule must have (transposition swaps the row and
column patterns; a power-of-two scale and a permutation of lines change
nothing), and synthetic tensors with planted outlier lines.
"""
import numpy as np
import pytest

import oracle
from synth import workloads as W

THRESHOLD = 8.0


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Exact bf16 bit patterns of fp32 values that bf16 represents."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    assert np.all(b & 0xFFFF == 0)
    return (b >> 16).astype(np.uint16)


def scores(t):
    return oracle.line_scores(t, oracle.ROWS, 64), oracle.line_scores(t, oracle.COLS, 64)


def test_hand_case_ratios():
    # 8 rows x 64 columns; row r = s_r * (+1, -1, +1, ...). A row's 64 values
    # are +-s_r: mean 0, population variance s_r^2. Column c holds the 8
    # values s_r * sign_c: the same variance for every column.
    s = np.array([1, 1, 1, 1, 1, 1, 1, 4], dtype=np.float32)
    sign = np.where(np.arange(64) % 2 == 0, 1.0, -1.0).astype(np.float32)
    t = bf16_bits(s[:, None] * sign[None, :])
    rs, cs = scores(t)
    assert np.array_equal(rs, np.array([1, 1, 1, 1, 1, 1, 1, 16], dtype=np.float64))
    # column values {1 x7, 4}: mean 11/8, E[x^2] = 23/8, variance 23/8 - 121/64 = 63/64
    assert np.all(cs == 63.0 / 64.0)
    # r_rows = 16 / 1, r_cols = 1
    assert oracle.classify_pattern(rs, cs, 8.0) == "R"
    assert oracle.classify_pattern(rs, cs, 16.0) == "R"
    assert oracle.classify_pattern(rs, cs, 16.5) == "N"
    # the transposed tensor: the same lines, now columns
    rt, ct = scores(np.ascontiguousarray(t.T))
    assert oracle.classify_pattern(rt, ct, 8.0) == "C"


def test_lower_median_and_degenerate_axes():
    # lower median of 4 values is the 2nd smallest
    assert oracle.classify_pattern([1, 2, 3, 16], [1, 1], 8.0) == "R"      # 16 / 2 = 8
    assert oracle.classify_pattern([1, 2, 3, 15.9], [1, 1], 8.0) == "N"    # 7.95
    assert oracle.classify_pattern([0, 0, 0, 1], [1, 1], 8.0) == "R"       # zero median
    assert oracle.classify_pattern([0, 0, 0, 0], [0, 0], 8.0) == "N"       # all zero
    assert oracle.classify_pattern([1, 1], [1, 1, 100], 8.0) == "C"


def planted(pattern, rows, cols, seed, frac=0.01, factor=50.0, name="X"):
    dim = rows if pattern == "R" else cols
    spec = W.TensorSpec(name, rows, cols, pattern, max(1, round(frac * dim)) if pattern != "N" else 0,
                        factor)
    return spec.make(seed)


@pytest.mark.parametrize("pattern", ["R", "C", "N"])
@pytest.mark.parametrize("shape", [(512, 1024), (2048, 384), (300, 4100)])
@pytest.mark.parametrize("seed", [0, 1])
def test_planted_patterns(pattern, shape, seed):
    t = planted(pattern, *shape, seed)
    assert oracle.classify_pattern(*scores(t), THRESHOLD) == pattern


@pytest.mark.parametrize("name,sigma_factor", [("X", 30.0), ("GY", 100.0), ("W", 50.0)])
def test_invariances(name, sigma_factor):
    rng = np.random.default_rng(7)
    t = planted("R", 1024, 768, 3, frac=0.005, factor=sigma_factor, name=name)
    base = oracle.classify_pattern(*scores(t), THRESHOLD)
    assert base == "R"
    # transposition swaps the patterns
    assert oracle.classify_pattern(*scores(np.ascontiguousarray(t.T)), THRESHOLD) == "C"
    # a power-of-two scale: x 8 is exponent + 3 on every nonzero value (no
    # value is near the top of the range; zeros stay zero)
    nz = (t & 0x7FFF) != 0
    t2 = np.where(nz, t.astype(np.uint32) + (3 << 7), t).astype(np.uint16)
    assert oracle.classify_pattern(*scores(t2), THRESHOLD) == base
    # a permutation of the rows (beyond the probe, the column scores see other
    # rows; the row pattern stays)
    perm = rng.permutation(t.shape[0])
    assert oracle.classify_pattern(*scores(np.ascontiguousarray(t[perm])), THRESHOLD) == base
