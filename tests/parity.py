"""Comparison rules between GPU results and the oracle.

The GEMM bar: relative Frobenius error <= 1e-5 against the fp64 oracle on the
same dequantized operands, and every bf16 output within 1 bf16 ulp.

Reading of the 1-ulp bar. The library accumulates in fp32 (the matrix cores'
accumulator) and rounds once to bf16. Rounding alone leaves the bf16 output
within half an ulp of the fp32 value, so the output is within 1 ulp of the
fp64 reference wherever the fp32 accumulation error is at most half an ulp.
The accumulation error is bounded per element by

    gamma = u * (walk + C_INT * sum|ab| + (72 + k_inner / 8) * rmax),
    u = 2^-24,

where walk and rmax are the oracle's running-error terms (the partial sums an
accumulator holds when it adds the products in contraction order, 32 FP4 or
8 bf16 products at a time at most, also when the contraction is cut into
contiguous parts added afterwards: first-order recursive-summation bound),
C_INT * sum|ab| covers the roundings inside one matrix-core step, and the
rmax term the additions after the contraction loop (up to 4 parts of a tile
split along K, up to 64 partial sums of the outlier product, the scatter-add,
and an inner outlier term of rank k_inner added step by step to the finished
residual).

Every element must be within gamma of the reference in fp32. In bf16, an
element is "strict" where gamma <= ulp/2: it must be within 1 ulp; elsewhere
(cancellation: the reference is small next to the partial sums) it must be
within ulp + gamma; where the reference is 0 the output must be within gamma.
The maximum error in ulps over the strict elements, the strict and loose
counts and the number of elements beyond 1 ulp are returned for the log.
"""
import numpy as np

U = 2.0 ** -24
C_INT = 4


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


def gamma(absC, walk, rmax, k_inner=0) -> np.ndarray:
    """fp32 accumulation-error bound per element (module docstring)."""
    return U * (walk + C_INT * absC + (72 + k_inner / 8) * rmax)


def gamma_of(ref: dict) -> np.ndarray:
    """The bound for an oracle pipeline result (oracle.pipeline.gemm)."""
    return gamma(ref["absC"], ref["walk"], ref["rmax"], ref.get("k_inner", 0))


def check_f32(C: np.ndarray, ref: np.ndarray, g: np.ndarray, tag=""):
    C = C.astype(np.float64)
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(C - ref) / (nref if nref > 0 else 1.0)
    assert rel <= 1e-5, f"{tag}: relative Frobenius error {rel:.3e}"
    err = np.abs(C - ref)
    bad = err > g
    assert not bad.any(), (f"{tag}: {bad.sum()} elements beyond the accumulation bound "
                           f"(worst err/gamma {float(np.max(err / np.maximum(g, 1e-300))):.3f})")
    return rel


def check_bf16(C_bits: np.ndarray, ref: np.ndarray, g: np.ndarray, tag="") -> dict:
    C = bf16_to_f32(C_bits).astype(np.float64)
    u = ulp_bf16(ref)
    err = np.abs(C - ref)
    zero = ref == 0
    strict = (g <= u / 2) & ~zero
    loose = ~strict & ~zero
    over = err[strict] > u[strict]
    assert not over.any(), f"{tag}: {int(over.sum())} strict elements beyond 1 bf16 ulp"
    assert not (err[loose] > u[loose] + g[loose]).any(), f"{tag}: elements beyond ulp + gamma"
    assert not (np.abs(C[zero]) > g[zero]).any(), f"{tag}: nonzero where the reference is 0"
    nref = np.linalg.norm(ref)
    ulps = err[~zero] / u[~zero]
    return {
        "rel": float(np.linalg.norm(C - ref) / (nref if nref > 0 else 1.0)),
        "strict": int(strict.sum()),
        "loose": int(loose.sum()),
        "max_ulp_strict": float(np.max(err[strict] / u[strict])) if strict.any() else 0.0,
        "beyond_1ulp": int((ulps > 1.0).sum()),
        "max_ulp": float(ulps.max()) if ulps.size else 0.0,
    }


def describe(stats: dict) -> str:
    n = stats["strict"] + stats["loose"]
    return (f"rel bf16 {stats['rel']:.2e}, strict (1 ulp) {stats['strict']}/{n} elements, "
            f"max {stats['max_ulp_strict']:.3f} ulp there; {stats['beyond_1ulp']} beyond 1 ulp "
            f"overall (max {stats['max_ulp']:.3f})")
