"""Seeded synthetic bf16 operands (shared by the GPU tests, the oracle tests,
the benchmark and the smoke check).

Only input generation lives here; none of the method's arithmetic does. The
generator and the workload shapes are described in ``synth.c`` and
``workloads.py``.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it first (python synth/build.py "
                "or __graft_entry__.build())")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_pick_lines.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_void_p]
        lib.synth_pick_lines.restype = ctypes.c_int
        lib.synth_fill_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64,
                                        ctypes.c_double, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_double]
        lib.synth_fill_bf16.restype = ctypes.c_int
        _lib = lib
    return _lib


def pick_lines(seed: int, stream: int, dim: int, n: int) -> np.ndarray:
    """n distinct indices in [0, dim), ascending (int64)."""
    out = np.zeros(max(n, 1), dtype=np.int64)
    rc = _load().synth_pick_lines(seed, stream, dim, n, out.ctypes.data)
    if rc != 0:
        raise ValueError(f"pick_lines: bad sizes dim={dim} n={n}")
    return out[:n].copy()


def fill_bf16(rows: int, cols: int, seed: int, stream: int, sigma: float,
              line_axis: int = -1, lines=None, factor: float = 1.0,
              out: np.ndarray = None) -> np.ndarray:
    """bf16 bit patterns (uint16) of a [rows, cols] tensor; see synth.c."""
    if out is None:
        out = np.empty((rows, cols), dtype=np.uint16)
    assert out.dtype == np.uint16 and out.shape == (rows, cols) and out.flags.c_contiguous
    lines = np.ascontiguousarray(np.asarray([] if lines is None else lines, dtype=np.int64))
    rc = _load().synth_fill_bf16(out.ctypes.data, rows, cols, cols, seed, stream, sigma,
                                 line_axis, lines.ctypes.data if lines.size else None,
                                 lines.size, factor)
    if rc != 0:
        raise ValueError("fill_bf16: bad arguments")
    return out
