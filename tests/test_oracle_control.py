"""Pins of the per-block runtime control oracle (6Bit-Diffusion page, Methodology B.1-B.3).

The stability statistic E is checked against closed forms (identical, doubled and
hand-summed deltas, the zero cases) and exact invariances; the decision rule against a
hand-worked table of sequences (tests/golden/control.json) whose E and Gamma are dyadic,
so every accumulation and comparison in it is exact.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import control

GOLD = os.path.join(os.path.dirname(__file__), "golden", "control.json")


def test_stability_closed_forms():
    d2 = np.array([1.0, -2.0, 3.0, -4.0], np.float32)
    assert control.stability(d2, d2) == 0.0
    assert control.stability(2 * d2, d2) == 1.0                      # sum|d2| / sum|d2|
    assert control.stability(np.array([1.0, -2.0, 3.0, -3.5], np.float32), d2) == 0.05  # 0.5 / 10
    assert control.stability(-d2, d2) == 2.0                         # sum|2 d2| / sum|d2|
    z = np.zeros(4, np.float32)
    assert control.stability(z, z) == 0.0
    assert math.isinf(control.stability(d2, z))
    assert control.stability(z, d2) == 1.0


def test_stability_invariances():
    g = np.random.default_rng(5)
    d1 = g.standard_normal(1000).astype(np.float32)
    d2 = (d1 + 0.01 * g.standard_normal(1000)).astype(np.float32)
    e = control.stability(d1, d2)
    assert 0.0 < e < 0.05
    for k in (-3, 4):  # power-of-two scaling is exact in every sum
        s = np.float32(2.0 ** k)
        assert control.stability(d1 * s, d2 * s) == e
    assert control.stability(-d1, -d2) == e
    perm = g.permutation(1000)
    assert control.stability(d1[perm], d2[perm]) == pytest.approx(e, rel=1e-13)


def _num(v):
    return float("inf") if v == "inf" else v


def test_decision_table():
    gold = json.load(open(GOLD))
    p = control.Params(**gold["params"])
    for seq in gold["sequences"]:
        st = control.State()
        for i, s in enumerate(seq["steps"]):
            skip, bits, st = control.step(st, p, _num(s["e"]), s["gamma"], s.get("n_out"), s.get("channels"))
            where = f'{seq["name"]}, step {i}'
            assert (skip, bits) == (s["skip"], s["bits"]), where
            assert (st.skips, st.drift) == (s["skips"], s["drift"]), where


def test_no_skips_allowed():
    p = control.Params(max_skips=0)
    skip, bits, st = control.step(control.State(), p, 0.0, 0.0)
    assert not skip and bits == p.bits_lo and st.skips == 0
