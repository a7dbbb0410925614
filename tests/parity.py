"""Comparison rules between GPU results and the oracle.

bf16/fp32 outputs follow the GEMM bar: relative Frobenius error <= 1e-5,
and every element within the fp32 accumulation bound gamma of the fp64
reference; bf16 outputs additionally within 1 bf16 ulp where gamma <= ulp/2
(strict), ulp + gamma elsewhere, and |C| <= gamma where the reference is 0.

gamma(i, j) = (K/16 + 64) * 2^-24 * sum_t |a_it * b_tj|: one fp32 rounding per
bf16 MFMA step of 16 (the FP4 path takes 64 per step, so this is a 4x margin)
plus up to 64 partial sums, relative to the absolute sum of the products.
"""
import numpy as np


def bf16_to_f32(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126)
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def gamma(absC: np.ndarray, K: int) -> np.ndarray:
    return (K / 16 + 64) * 2.0 ** -24 * absC


def check_f32(C: np.ndarray, ref: np.ndarray, absC: np.ndarray, K: int, tag=""):
    C = C.astype(np.float64)
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(C - ref) / (nref if nref > 0 else 1.0)
    assert rel <= 1e-5, f"{tag}: relative Frobenius error {rel:.3e}"
    g = gamma(absC, K)
    bad = np.abs(C - ref) > g
    assert not bad.any(), f"{tag}: {bad.sum()} elements beyond the accumulation bound"
    return rel


def check_bf16(C_bits: np.ndarray, ref: np.ndarray, absC: np.ndarray, K: int, tag=""):
    C = bf16_to_f32(C_bits).astype(np.float64)
    g = gamma(absC, K)
    u = ulp_bf16(ref)
    err = np.abs(C - ref)
    strict = g <= u / 2
    assert not (err[strict] > u[strict]).any(), \
        f"{tag}: {(err[strict] > u[strict]).sum()} elements beyond 1 bf16 ulp"
    loose = ~strict
    assert not (err[loose] > u[loose] + g[loose]).any(), f"{tag}: elements beyond ulp + gamma"
    zero = ref == 0
    assert not (np.abs(C[zero]) > g[zero]).any(), f"{tag}: nonzero where the reference is 0"
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(C - ref) / (nref if nref > 0 else 1.0)
    return rel, int(loose.sum())
