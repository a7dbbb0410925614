"""Pins of the oracle's FOID (variance of the first 64 elements of each
candidate line, top-k, ties to the lower index) against exact rational
brute force and the planted-outlier invariant."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


def to_bf16(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def brute_force(t_f32, axis, k, probe=64):
    """Exact population variance with Fractions, full sort by (-var, index)."""
    lines = t_f32 if axis == oracle.ROWS else t_f32.T
    P = min(probe, lines.shape[1])
    scored = []
    for l, line in enumerate(lines):
        xs = [Fraction(float(v)) for v in line[:P]]
        mu = sum(xs) / P
        var = sum((x - mu) ** 2 for x in xs) / P
        scored.append((-var, l))
    scored.sort()
    return sorted(l for _, l in scored[:k])


@pytest.mark.parametrize("axis", [0, 1])
def test_integer_data_with_ties(axis):
    """Integer-valued data with a power-of-two probe: the fp64 mean and
    variance are then exact, so ties are frequent and the tie-break to the
    lower index is exercised."""
    rng = np.random.default_rng(11 + axis)
    for trial in range(30):
        rows, cols = rng.integers(3, 90), rng.integers(3, 90)
        t = rng.integers(-3, 4, size=(rows, cols)).astype(np.float32)
        ncand, length = (rows, cols) if axis == 0 else (cols, rows)
        probe = 64 if length >= 64 else 1 << int(np.log2(length))
        k = int(rng.integers(1, ncand + 1))
        got = oracle.foid(to_bf16(t), axis, k, probe=probe)
        assert list(got) == brute_force(t, axis, k, probe), (trial, rows, cols, k)


@pytest.mark.parametrize("axis", [0, 1])
def test_random_data(axis):
    rng = np.random.default_rng(21 + axis)
    for trial in range(10):
        rows, cols = rng.integers(40, 130), rng.integers(40, 130)
        t = (rng.standard_normal((rows, cols)) * rng.uniform(0.5, 2, size=(1, cols))).astype(np.float32)
        t = (to_bf16(t).astype(np.uint32) << 16).view(np.float32)
        k = int(rng.integers(1, 20))
        got = oracle.foid(to_bf16(t), axis, k)
        assert list(got) == brute_force(t, axis, k)


def test_only_the_probe_matters():
    rng = np.random.default_rng(5)
    t = rng.standard_normal((200, 96)).astype(np.float32)
    a = oracle.foid(to_bf16(t), oracle.COLS, 10)
    t2 = t.copy()
    t2[64:, :] = rng.standard_normal((136, 96)) * 1000     # beyond the first 64 rows
    assert np.array_equal(oracle.foid(to_bf16(t2), oracle.COLS, 10), a)
    t3 = t.copy()
    t3[:64, 5] *= 100                                         # inside the probe
    assert 5 in oracle.foid(to_bf16(t3), oracle.COLS, 10)


def test_probe_clamped_to_line_length():
    rng = np.random.default_rng(6)
    t = rng.integers(-4, 5, size=(16, 30)).astype(np.float32)   # columns shorter than 64
    assert list(oracle.foid(to_bf16(t), oracle.COLS, 7)) == brute_force(t, oracle.COLS, 7, 64)
    assert list(oracle.foid(to_bf16(t), oracle.ROWS, 7, probe=8)) == brute_force(t, oracle.ROWS, 7, 8)


def test_rows_of_t_equal_cols_of_transpose():
    rng = np.random.default_rng(8)
    t = to_bf16(rng.standard_normal((77, 140)))
    assert np.array_equal(oracle.foid(t, oracle.ROWS, 9), oracle.foid(np.ascontiguousarray(t.T), oracle.COLS, 9))


@pytest.mark.parametrize("n_planted,k", [(8, 16), (20, 20), (41, 64), (143, 64)])
def test_planted_lines(n_planted, k):
    """Lines scaled x50 have ~2500x the variance: with k >= #planted every
    planted line is chosen; with k <= #planted only planted lines are."""
    cols = 4096 if n_planted > 20 else 512
    lines = synth.pick_lines(0, 1, cols, n_planted)
    t = synth.fill_bf16(64, cols, 0, 1, 1.0, 1, lines, 50.0)
    got = set(oracle.foid(t, oracle.COLS, k).tolist())
    planted = set(lines.tolist())
    if k >= n_planted:
        assert planted <= got
    else:
        assert got <= planted


def test_invalid_arguments():
    t = np.zeros((4, 4), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.foid(t, oracle.ROWS, 5)          # k > candidates
    with pytest.raises(ValueError):
        oracle.foid(t, oracle.ROWS, 0)
