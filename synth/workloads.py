"""The synthetic GEMM workloads: operand shapes, value distributions and
planted outlier lines, plus the AdaHOP GEMM calls made on them.

Shapes are those of the linear layers named in the workload descriptions
(Llama3.2-1B hidden 2048 / FFN 8192; Llama3.1-8B hidden 4096 / FFN 14336,
seq 4096 x batch). Values: entries N(0, sigma^2) with sigma 1 for activations
X, 0.02 for weights W and 1e-3 for output gradients GY. A Column-wise operand
has round(p * cols) columns scaled by a factor, a Row-wise one round(p * rows)
rows; a None operand has no planted lines.

Streams: X = 1, W = 2, GY = 3 (the planted-line choice uses 16 + stream).
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from . import fill_bf16, pick_lines

STREAM = {"X": 1, "W": 2, "GY": 3}
SIGMA = {"X": 1.0, "W": 0.02, "GY": 1e-3}


@dataclass
class TensorSpec:
    name: str                 # "X", "W" or "GY"
    rows: int
    cols: int
    pattern: str = "N"        # "R" (rows planted), "C" (columns planted), "N"
    n_lines: int = 0
    factor: float = 1.0

    @property
    def stream(self) -> int:
        return STREAM[self.name]

    @property
    def sigma(self) -> float:
        return SIGMA[self.name]

    def lines(self, seed: int) -> np.ndarray:
        if self.pattern == "N" or self.n_lines == 0:
            return np.zeros(0, dtype=np.int64)
        dim = self.rows if self.pattern == "R" else self.cols
        return pick_lines(seed, self.stream, dim, self.n_lines)

    def make(self, seed: int, out: np.ndarray = None) -> np.ndarray:
        axis = {"R": 0, "C": 1, "N": -1}[self.pattern]
        return fill_bf16(self.rows, self.cols, seed, self.stream, self.sigma, axis,
                         self.lines(seed), self.factor, out=out)


@dataclass
class CallSpec:
    op: str                   # "FWD", "DGRAD", "WGRAD"
    lhs: str
    rhs: str
    pat_lhs: str              # storage-frame pattern of lhs: "N", "R", "C"
    pat_rhs: str
    route: Optional[str] = None   # None = chosen by the pattern-pair router
    k: int = 64


@dataclass
class Workload:
    name: str
    T: int
    Din: int
    Dout: int
    tensors: Dict[str, TensorSpec]
    calls: List[CallSpec] = field(default_factory=list)


def _n(p: float, dim: int) -> int:
    return int(round(p * dim))


def tiny_fwd() -> Workload:
    """Y = X W^T, X [256,512] with 8 columns x50, W [512,512]; IHT route, then
    inner outlier extraction of rank 16."""
    T, Din, Dout = 256, 512, 512
    t = {"X": TensorSpec("X", T, Din, "C", 8, 50.0), "W": TensorSpec("W", Dout, Din)}
    calls = [CallSpec("FWD", "X", "W", "C", "N", None, 64),
             CallSpec("FWD", "X", "W", "C", "N", "OE_INNER", 16)]
    return Workload("tiny_fwd_256x512x512", T, Din, Dout, t, calls)


def l32_1b_up_fwd() -> Workload:
    """Llama3.2-1B FFN up-projection forward, X [16384,2048] with 1% of columns
    x30, W [8192,2048]."""
    T, Din, Dout = 16384, 2048, 8192
    t = {"X": TensorSpec("X", T, Din, "C", _n(0.01, Din), 30.0),
         "W": TensorSpec("W", Dout, Din)}
    return Workload("llama3.2-1b_up_fwd_16384x8192x2048", T, Din, Dout, t,
                    [CallSpec("FWD", "X", "W", "C", "N")])


def l31_8b_down_wgrad() -> Workload:
    """Llama3.1-8B down_proj weight gradient dW = GY^T X over 32768 tokens;
    GY [32768,4096] with 0.5% of rows x100, X [32768,14336] with 1% of
    columns x50; outlier extraction of rank 64 on X's columns."""
    T, Din, Dout = 32768, 14336, 4096
    t = {"GY": TensorSpec("GY", T, Dout, "R", _n(0.005, T), 100.0),
         "X": TensorSpec("X", T, Din, "C", _n(0.01, Din), 50.0)}
    return Workload("llama3.1-8b_down_wgrad_4096x14336x32768", T, Din, Dout, t,
                    [CallSpec("WGRAD", "GY", "X", "R", "C", None, 64)])


def l31_8b_gateup_fwd_dgrad() -> Workload:
    """Llama3.1-8B gate/up projection forward and input gradient; X [32768,4096]
    with 1% of columns x50, W [14336,4096], GY [32768,14336] with no pattern."""
    T, Din, Dout = 32768, 4096, 14336
    t = {"X": TensorSpec("X", T, Din, "C", _n(0.01, Din), 50.0),
         "W": TensorSpec("W", Dout, Din),
         "GY": TensorSpec("GY", T, Dout)}
    return Workload("llama3.1-8b_gateup_fwd_dgrad_32768x14336x4096", T, Din, Dout, t,
                    [CallSpec("FWD", "X", "W", "C", "N"),
                     CallSpec("DGRAD", "GY", "W", "N", "N")])


def l31_8b_oproj_triplet(bs: int) -> Workload:
    """Llama3.1-8B o_proj forward, input gradient and weight gradient at
    4096 x bs tokens; X with 1% of columns x50, GY with 0.5% of rows x100."""
    T, Din, Dout = 4096 * bs, 4096, 4096
    t = {"X": TensorSpec("X", T, Din, "C", _n(0.01, Din), 50.0),
         "W": TensorSpec("W", Dout, Din),
         "GY": TensorSpec("GY", T, Dout, "R", _n(0.005, T), 100.0)}
    calls = [CallSpec("FWD", "X", "W", "C", "N"),
             CallSpec("DGRAD", "GY", "W", "R", "N", None, 64),
             CallSpec("WGRAD", "GY", "X", "R", "C", None, 64)]
    return Workload(f"llama3.1-8b_oproj_triplet_bs{bs}", T, Din, Dout, t, calls)


ALL = {
    "tiny": tiny_fwd,
    "l1b_up": l32_1b_up_fwd,
    "l8b_down_wgrad": l31_8b_down_wgrad,
    "l8b_gateup": l31_8b_gateup_fwd_dgrad,
}
