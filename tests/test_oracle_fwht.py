"""Pins of the oracle's 32-point IHT block transform against the closed form
of the Sylvester-Hadamard matrix, hand-derived IHT+MXFP4 blocks, and the
invariance of the product under the inner rotation."""
from decimal import Decimal, getcontext

import numpy as np

import oracle
from conftest import read_golden


def sylvester(n):
    """H[i][j] = (-1)^popcount(i & j), integers."""
    i = np.arange(n)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def test_sylvester_orthogonal():
    H = sylvester(32)
    assert np.array_equal(H @ H.T, 32 * np.eye(32, dtype=np.int64))


def test_inv_sqrt32_is_nearest_fp32():
    getcontext().prec = 60
    exact = Decimal(1) / Decimal(32).sqrt()
    f = np.float32(1.0 / np.sqrt(32.0))
    assert f.view(np.uint32) == 0x3E3504F3
    lo = np.nextafter(f, np.float32(0)); hi = np.nextafter(f, np.float32(1))
    d = abs(Decimal(float(f)) - exact)
    assert d < abs(Decimal(float(lo)) - exact) and d < abs(Decimal(float(hi)) - exact)


def test_one_hot_columns_bit_exact():
    H = sylvester(32)
    c = np.float32(1.0 / np.sqrt(32.0))
    for j in range(32):
        e = np.zeros(32, dtype=np.float32); e[j] = 1
        y = oracle.fwht32(e)
        assert np.array_equal(y, (H[:, j] * c).astype(np.float32)), j


def test_matches_dense_hadamard():
    rng = np.random.default_rng(1)
    H = sylvester(32).astype(np.float64) / np.sqrt(32.0)
    for _ in range(500):
        x = (rng.standard_normal(32) * rng.choice([1e-3, 1, 50])).astype(np.float32)
        y = oracle.fwht32(x).astype(np.float64)
        ref = H @ x.astype(np.float64)
        assert np.max(np.abs(y - ref)) <= 2.0 ** -20 * max(np.max(np.abs(ref)), 1e-30) * 8


def test_involution_and_energy():
    rng = np.random.default_rng(2)
    for _ in range(200):
        x = rng.standard_normal(32).astype(np.float32)
        y = oracle.fwht32(x)
        z = oracle.fwht32(y)
        assert np.allclose(z, x, rtol=0, atol=1e-5 * np.max(np.abs(x)))
        assert abs(np.linalg.norm(y.astype(np.float64)) - np.linalg.norm(x.astype(np.float64))) \
            <= 1e-5 * np.linalg.norm(x.astype(np.float64))


def test_inner_rotation_keeps_product():
    """(A H)(H^T B) = A B: rotating A's rows and B's columns blockwise along
    the contraction dim (the oracle's transform) leaves the product, up to
    the fp32 rounding of the rotated values."""
    rng = np.random.default_rng(3)
    m, K, n = 8, 128, 6
    A = rng.standard_normal((m, K)).astype(np.float32)
    B = rng.standard_normal((K, n)).astype(np.float32)
    Ar = np.stack([np.concatenate([oracle.fwht32(A[i, b:b + 32]) for b in range(0, K, 32)])
                   for i in range(m)])
    Br = np.stack([np.concatenate([oracle.fwht32(B[b:b + 32, j]) for b in range(0, K, 32)])
                   for j in range(n)], axis=1)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    rot = Ar.astype(np.float64) @ Br.astype(np.float64)
    assert np.max(np.abs(rot - exact)) <= 1e-5 * np.max(np.abs(exact))
    # A wrong sign or stride would break the identity by O(1).
    Hd = np.kron(np.eye(K // 32), sylvester(32).astype(np.float64) / np.sqrt(32))
    assert np.allclose(Ar.astype(np.float64), A.astype(np.float64) @ Hd.T, atol=1e-5)


def _parse_iht():
    out, cur = [], None
    for ln in read_golden("iht_blocks.txt"):
        key, *rest = ln.split()
        if key == "onehot":
            cur = {"j": int(rest[0]), "v": float(rest[1])}
            out.append(cur)
        elif key == "scale":
            cur["scale"] = int(rest[0])
        elif key == "codes":
            cur["codes"] = bytes(int(x, 16) for x in rest)
    return out


def test_hand_derived_iht_blocks():
    cases = _parse_iht()
    assert len(cases) == 4
    for c in cases:
        src = np.zeros((1, 32), dtype=np.float32)
        src[0, c["j"]] = c["v"]
        bf = (src.view(np.uint32) >> 16).astype(np.uint16)
        codes, scales, _ = oracle.iht_quant(bf, oracle.COLS, 32)
        assert int(scales[0, 0]) == c["scale"]
        assert bytes(codes[0]) == c["codes"], bytes(codes[0]).hex()
        # Same block down a column (contraction along rows).
        codes2, scales2, _ = oracle.iht_quant(np.ascontiguousarray(bf.T), oracle.ROWS, 32)
        assert bytes(codes2[0]) == c["codes"] and int(scales2[0, 0]) == c["scale"]
