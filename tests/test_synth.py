"""The seeded input generator: determinism, counter-based regeneration,
distribution and planted lines."""
import numpy as np

import synth
from synth import workloads


def f32(x):
    return (x.astype(np.uint32) << 16).view(np.float32)


def test_deterministic_and_seeded():
    a = synth.fill_bf16(64, 96, 3, 1, 1.0)
    b = synth.fill_bf16(64, 96, 3, 1, 1.0)
    c = synth.fill_bf16(64, 96, 4, 1, 1.0)
    d = synth.fill_bf16(64, 96, 3, 2, 1.0)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)


def test_counter_based_prefix():
    """Element (r, c) depends on r*cols + c only: a taller tensor with the same
    width starts with the same rows."""
    a = synth.fill_bf16(10, 33, 0, 1, 1.0)
    b = synth.fill_bf16(25, 33, 0, 1, 1.0)
    assert np.array_equal(a, b[:10])


def test_distribution():
    x = f32(synth.fill_bf16(512, 512, 0, 2, 0.02)).astype(np.float64)
    assert abs(x.mean()) < 0.001 and abs(x.std() - 0.02) < 0.0005
    assert np.all(np.isfinite(x))


def test_planted_lines():
    lines = synth.pick_lines(0, 1, 4096, 41)
    assert lines.size == 41 and np.all(np.diff(lines) > 0) and lines.max() < 4096
    x = f32(synth.fill_bf16(256, 4096, 0, 1, 1.0, 1, lines, 50.0)).astype(np.float64)
    std = x.std(axis=0)
    assert np.all(std[lines] > 30) and np.delete(std, lines).max() < 2


def test_workload_shapes():
    wl = workloads.l31_8b_down_wgrad()
    assert (wl.T, wl.Din, wl.Dout) == (32768, 14336, 4096)
    assert wl.tensors["GY"].n_lines == 164 and wl.tensors["X"].n_lines == 143
    t = workloads.tiny_fwd()
    assert t.tensors["X"].n_lines == 8 and t.calls[1].route == "OE_INNER" and t.calls[1].k == 16
    assert workloads.l31_8b_oproj_triplet(8).tensors["GY"].n_lines == 164
