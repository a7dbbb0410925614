"""Pins of the oracle's MXFP4 encoder and decoder (E2M1 elements, E8M0 scale
per 32-element block) against the OCP MX v1.0 grid, hand-derived blocks, an
exhaustive nearest-grid search and the format's error bounds."""
import math

import numpy as np
import pytest

import oracle
from conftest import read_golden


def golden_grid():
    return {int(c, 16): float(v) for c, v in (ln.split() for ln in read_golden("e2m1_grid.txt"))}


def test_decode_grid_matches_ocp_table():
    grid = golden_grid()
    assert len(grid) == 16
    for code, val in grid.items():
        got = oracle.e2m1_value(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    mags = sorted({abs(v) for v in grid.values()})
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _nearest_even(v):
    """Independent rounding onto the E2M1 magnitude grid: the nearest grid
    value, an exact tie going to the code whose mantissa bit is 0, values
    beyond 6 saturating."""
    grid = [abs(golden_grid()[c]) for c in range(8)]
    best = None
    for code, g in enumerate(grid):
        d = abs(v - g)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0 and best[1] % 2 == 1):
            best = (d, code)
    return best[1]


def test_magnitude_rounding_exhaustive_bf16():
    """Every non-negative finite bf16 value, at scale exponents across the
    range, rounds as the independent nearest-grid search says."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    checked = 0
    for s in (-127, -30, -1, 0, 1, 30, 127):
        v = np.ldexp(vals, -s)
        # Only the band where rounding is non-trivial needs the slow search;
        # below 0.25 everything is code 0 and above 6 everything saturates.
        for x in v[(v > 0.2) & (v < 6.5)]:
            assert oracle.e2m1_magnitude(x) == _nearest_even(x), x
            checked += 1
        assert all(oracle.e2m1_magnitude(x) == 0 for x in v[v <= 0.2][::97])
        assert all(oracle.e2m1_magnitude(x) == 7 for x in v[v >= 6.5][::97])
    assert checked > 1000


def _parse_blocks(name):
    blocks, cur = {}, None
    for ln in read_golden(name):
        key, *rest = ln.split()
        if key == "block":
            cur = blocks.setdefault(rest[0], {})
        elif key == "values":
            cur["values"] = np.array([float(x) for x in rest], dtype=np.float32)
        elif key == "values_pow2":
            cur["values"] = np.ldexp(blocks[rest[0]]["values"], int(rest[1])).astype(np.float32)
        elif key == "scale":
            cur["scale"] = int(rest[0])
        elif key == "codes":
            cur["codes"] = bytes(int(x, 16) for x in rest)
    return blocks


def test_hand_derived_blocks():
    blocks = _parse_blocks("mx_blocks.txt")
    assert len(blocks) >= 8
    for name, b in blocks.items():
        assert b["values"].shape == (32,), name
        codes, scale = oracle.mx_block(b["values"])
        assert scale == b["scale"], (name, scale)
        assert bytes(codes) == b["codes"], (name, bytes(codes).hex())


def _decode_block(codes, scale):
    grid = golden_grid()
    out = []
    for byte in codes:
        for nib in (byte & 15, byte >> 4):
            out.append(grid[nib] * 2.0 ** (scale - 127))
    return np.array(out)


def test_block_invariants_random():
    rng = np.random.default_rng(7)
    for trial in range(2000):
        y = (rng.standard_normal(32) * 10.0 ** rng.uniform(-30, 30)).astype(np.float32)
        if trial % 5 == 0:
            y[rng.integers(32)] *= 50
        codes, scale = oracle.mx_block(y)
        s = scale - 127
        amax = float(np.max(np.abs(y)))
        # The block's largest element lands in [4, 8) after scaling and gets
        # one of the two top codes.
        assert 4.0 <= amax / 2.0 ** s < 8.0
        deq = _decode_block(codes, scale)
        top = int(np.argmax(np.abs(y)))
        assert abs(deq[top]) >= 4 * 2.0 ** s
        # Half a grid step of at most 1 (x 2^s) below 6, up to 2 in the
        # saturating band.
        err = np.abs(y.astype(np.float64) - deq)
        band = np.abs(y) > 6 * 2.0 ** s
        assert np.all(err[~band] <= 1.0 * 2.0 ** s)
        assert np.all(err[band] <= 2.0 * 2.0 ** s)
        # Signs survive (zero magnitude keeps the sign bit).
        nibbles = np.array([(c >> (4 * h)) & 15 for c in codes for h in (0, 1)])
        assert np.all((nibbles >> 3) == np.signbit(y).astype(int))


def test_round_trip_every_code():
    """A block whose values are grid points x 2^s (with a 6 x 2^s element to
    fix the scale) encodes back to the same codes, for many scales."""
    grid = golden_grid()
    for s in (-127, -100, -7, -1, 0, 1, 9, 60, 125):
        codes_in = list(range(16)) * 2
        codes_in[0] = 7                     # 6 x 2^s fixes floor(log2 amax) - 2 = s
        vals = np.array([grid[c] * 2.0 ** s for c in codes_in], dtype=np.float32)
        codes, scale = oracle.mx_block(vals)
        assert scale == s + 127
        got = [(b >> (4 * h)) & 15 for b in codes for h in (0, 1)]
        assert got == codes_in, s


def test_tiny_scale_clamps_to_zero_byte():
    codes, scale = oracle.mx_block(np.full(32, 2.0 ** -140, dtype=np.float32))
    assert scale == 0
    assert not any(codes)
