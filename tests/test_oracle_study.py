"""Sign check of the relative-MSE improvement from IHT per outlier-pattern
pair (Fig. 3 of the AdaHOP pages: IHT helps only when its mixing direction
meets the outlier structure; improvement = (E_base - E_IHT) / E_base x 100).

Reading (the pages' Appendix D with the exact setup is not available): pairs
are named in the textbook frame C = A B; E = ||C_q - C_exact||^2 / ||C_exact||^2
with C_q the fp64 product of the dequantized MXFP4 operands (quantized along
the contraction dim, without or with the 32-point IHT) and C_exact the fp64
product of the bf16 operands; A, B are [512,512] N(0,1) with 1% of lines x50;
five seeds. IHT mixes A's columns and B's rows (the inner lines):
  - one operand with inner outliers, the other clean (CN, NR): above 20 %
    on every seed (measured minimum 22.9 %, NR);
  - one inner side and one outer side (CC, RR): positive on average (the
    outer lines dominate the error and IHT leaves them as they are);
  - no inner outliers (NN, NC, RN, RC): zero on average, since an orthogonal
    mix of an iid Gaussian block is iid Gaussian (RC, both outer, is noisy:
    a few intersection entries dominate the error);
  - inner outliers on both sides (CR): measured, not pinned: -11.6, -27.9,
    -12.8, +32.1, -38.2 % on seeds 0-4 (mean -11.7 %). Rotating both
    operands' outlier-hit blocks spreads each outlier over its 32 entries, so
    the ordinary values that share a block with an outlier are lost on both
    sides of every product that meets one; the sign depends on how the two
    sides' outlier blocks line up.
Magnitudes are not printed on the pages: the thresholds are ours."""
import numpy as np
import pytest

import oracle
import synth

N = 512
ONE_SIDED = {"CN", "NR"}
MIXED = {"CC", "RR"}
NEUTRAL = {"NN", "NC", "RN"}
NEUTRAL_NOISY = {"RC"}


def operand(pattern, seed, stream):
    axis = {"R": 0, "C": 1, "N": -1}[pattern]
    lines = synth.pick_lines(seed, stream, N, round(0.01 * N)) if pattern != "N" else None
    return synth.fill_bf16(N, N, seed, stream, 1.0, axis, lines, 50.0)


def improvement(pa, pb, seed):
    A = operand(pa, seed, 101)          # A [m][K], contraction along its columns
    B = operand(pb, seed, 102)          # B [K][n], contraction along its rows
    exact = oracle.bf16_to_f64(A) @ oracle.bf16_to_f64(B)
    e = {}
    for had in (0, 32):
        ac, as_, _ = oracle.iht_quant(A, oracle.COLS, had)
        bc, bs, _ = oracle.iht_quant(B, oracle.ROWS, had)
        Cq = oracle.dequant(ac, as_) @ oracle.dequant(bc, bs).T
        e[had] = np.sum((Cq - exact) ** 2) / np.sum(exact ** 2)
    return (e[0] - e[32]) / e[0] * 100


@pytest.mark.parametrize("pair", sorted(ONE_SIDED | MIXED | NEUTRAL | NEUTRAL_NOISY))
def test_improvement_sign(pair):
    vals = [improvement(pair[0], pair[1], s) for s in range(5)]
    if pair in ONE_SIDED:
        assert min(vals) > 20, vals
    elif pair in MIXED:
        assert np.mean(vals) > 10, vals
    elif pair in NEUTRAL:
        assert abs(np.mean(vals)) < 5, vals
    else:
        assert abs(np.mean(vals)) < 10, vals


def test_improvement_cr_recorded():
    # CR (inner outliers on both operands) is a measured result, not a pinned
    # sign: the mean over the five seeds is negative (-11.7 %), four seeds of
    # five below zero.
    vals = [improvement("C", "R", s) for s in range(5)]
    print("CR improvement per seed (%):", [round(v, 1) for v in vals])
    assert all(np.isfinite(vals)) and np.mean(vals) < 0 and sum(v < 0 for v in vals) == 4, vals


def test_rotation_along_the_wrong_axis_is_neutral():
    """Control: rotating along the outer dim instead (A's rows, B's columns)
    leaves the one-sided pairs without gain, so the positive result above is
    due to the inner direction."""
    A = operand("C", 0, 101)
    B = operand("N", 0, 102)
    exact = oracle.bf16_to_f64(A) @ oracle.bf16_to_f64(B)
    e = {}
    for had in (0, 32):
        # Quantize along K, but rotate along the outer dim by transposing around it.
        if had:
            Ar = np.concatenate([np.stack([oracle.fwht32(oracle.bf16_to_f64(A)[i:i + 32, j].astype(np.float32))
                                            for j in range(N)], axis=1) for i in range(0, N, 32)])
            u = Ar.astype(np.float32).view(np.uint32).astype(np.uint64)
            A_use = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)   # bf16, RNE
        else:
            A_use = A
        ac, as_, _ = oracle.iht_quant(A_use, oracle.COLS, 0)
        bc, bs, _ = oracle.iht_quant(B, oracle.ROWS, 0)
        deqA = oracle.dequant(ac, as_)
        if had:
            # undo the outer rotation in fp64 (orthonormal, symmetric)
            Hb = np.array([[(-1) ** bin(i & j).count("1") for j in range(32)] for i in range(32)]) / np.sqrt(32)
            deqA = np.concatenate([Hb @ deqA[i:i + 32] for i in range(0, N, 32)])
        Cq = deqA @ oracle.dequant(bc, bs).T
        e[had] = np.sum((Cq - exact) ** 2) / np.sum(exact ** 2)
    assert abs((e[0] - e[32]) / e[0] * 100) < 10
