"""Pins of the pattern-pair router. The routing figure of the AdaHOP pages
(Fig. 5) is not legible, so the rule is a reading; it is pinned by (1) the
routes the workload descriptions state, (2) Table 1's printed pair counts and
(3) the quantization-error behaviour the abstract and Fig. 2 describe, as
measured with the oracle's own quantizer (IHT where inner mixing helps, the
OE side that holds outer outlier lines otherwise)."""
import itertools

import numpy as np
import pytest

import oracle
import synth
from oracle import pipeline
from conftest import read_golden


def test_routes_stated_by_the_workloads():
    assert oracle.route("FWD", "C", "N") == "IHT"          # forward, CN
    assert oracle.route("DGRAD", "N", "N") == "IHT"        # input gradient, NN
    assert oracle.route("DGRAD", "R", "N") == "OE_LEFT"    # input gradient, GY Row-wise
    assert oracle.route("WGRAD", "R", "C") == "OE_RIGHT"   # weight gradient, RC
    # ... and its FOID runs over the columns of X (the rhs).
    assert oracle.scan_target("WGRAD", "OE_RIGHT") == (1, oracle.COLS)
    assert oracle.scan_target("DGRAD", "OE_LEFT") == (0, oracle.ROWS)


def test_table1_pairs():
    rows = [ln.split() for ln in read_golden("table1_pattern_pairs.txt")]
    assert len(rows) == 15
    per_model = {}
    for model, layers, pair, total, fwd, wgrad, dgrad in rows:
        layers, total, fwd, wgrad, dgrad = map(int, (layers, total, fwd, wgrad, dgrad))
        assert total == fwd + wgrad + dgrad
        s = per_model.setdefault(model, [layers, 0, 0, 0])
        s[1] += fwd; s[2] += wgrad; s[3] += dgrad
        # Every printed (GEMM, pair) runs in MXFP4 under the rule (no BF16 fallback).
        for op, count in (("FWD", fwd), ("WGRAD", wgrad), ("DGRAD", dgrad)):
            if count:
                assert oracle.route(op, pair[0], pair[1]) != "BF16", (op, pair)
    for model, (layers, fwd, wgrad, dgrad) in per_model.items():
        # 7 linear layers per block: forward and input-gradient columns are complete ...
        assert fwd == 7 * layers and dgrad == 7 * layers, model
        # ... the weight-gradient column is not: one printed row is missing.
        assert wgrad < 7 * layers, model
    # The weight-gradient pair absent from the printed rows and not declared
    # absent (RR, NR, CR) is CC, the one pair the rule sends to BF16.
    printed = {r[2] for r in rows}
    missing = {a + b for a, b in itertools.product("RCN", repeat=2)} - printed - {"RR", "NR", "CR"}
    assert missing == {"CC"}
    assert oracle.route("WGRAD", "C", "C") == "BF16"


def _operands(op, pl, pr, n=128, lines=4, seed=0):
    shapes = {"FWD": ((n, n), (n, n)), "DGRAD": ((n, n), (n, n)), "WGRAD": ((n, n), (n, n))}[op]
    out = []
    for t, (pat, shape) in enumerate(zip((pl, pr), shapes)):
        axis = {"R": 0, "C": 1, "N": -1}[pat]
        dim = shape[0] if pat == "R" else shape[1]
        li = synth.pick_lines(seed, 40 + t, dim, lines) if pat != "N" else None
        out.append(synth.fill_bf16(shape[0], shape[1], seed, 30 + t, 1.0, axis, li, 50.0))
    return out


def _exact(op, lhs, rhs):
    L, R = oracle.bf16_to_f64(lhs), oracle.bf16_to_f64(rhs)
    return {"FWD": L @ R.T, "DGRAD": L @ R, "WGRAD": L.T @ R}[op]


@pytest.mark.parametrize("op", ["FWD", "DGRAD", "WGRAD"])
def test_route_agrees_with_quantization_error(op):
    """For every storage pair the chosen route is the one the error model
    favours: an OE route beats IHT by 2x and the opposite OE; an IHT route is
    within 15% of the best one-sided OE. (BF16 cells are the reading that no
    one-sided route removes both operands' outer lines; not checked here.)"""
    n = 128
    for pl, pr in itertools.product("NRC", repeat=2):
        rule = oracle.route(op, pl, pr)
        if rule == "BF16":
            continue
        lhs, rhs = _operands(op, pl, pr, n)
        ex = _exact(op, lhs, rhs)
        err = {}
        for r in ("IHT", "OE_LEFT", "OE_RIGHT"):
            C = pipeline.gemm(op, lhs, rhs, n, n, n, pl, pr, route=r, k=8)["C"]
            err[r] = np.linalg.norm(C - ex) / np.linalg.norm(ex)
        if rule == "OE_LEFT":
            assert err["OE_LEFT"] < 0.5 * err["IHT"] and err["OE_LEFT"] < err["OE_RIGHT"], (pl, pr, err)
        elif rule == "OE_RIGHT":
            assert err["OE_RIGHT"] < 0.5 * err["IHT"] and err["OE_RIGHT"] < err["OE_LEFT"], (pl, pr, err)
        else:
            assert err["IHT"] <= 1.15 * min(err["OE_LEFT"], err["OE_RIGHT"]), (pl, pr, err)


def test_all_cells_defined():
    seen = set()
    for op in ("FWD", "DGRAD", "WGRAD"):
        for pl, pr in itertools.product("NRC", repeat=2):
            seen.add(oracle.route(op, pl, pr))
    assert seen == {"IHT", "OE_LEFT", "OE_RIGHT", "BF16"}
