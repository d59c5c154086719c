"""Pins of the CPU oracle (no GPU): every check in tests/oracle_pins.py, plus the hand-derived
worked example in tests/golden/tiny_attention.json."""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_attention.json")


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(oracle)


def _num(x):
    """Golden values are numbers or strings of the form 'a*ln(b)' / 'ln(b)'."""
    if isinstance(x, (int, float)):
        return float(x)
    s = x.replace(" ", "")
    coef = 1.0
    if "*" in s:
        c, s = s.split("*")
        coef = float(c)
    assert s.startswith("ln(") and s.endswith(")")
    return coef * math.log(float(s[3:-1]))


def _arr(rows):
    return np.array([[_num(x) for x in r] for r in rows])


@pytest.mark.parametrize("case", ["non_causal", "causal"])
def test_golden_tiny(case):
    g = json.load(open(GOLDEN))
    inp = g["inputs"]
    q, k, v, do = (_arr(inp[n]) for n in ("q", "k", "v", "do"))
    c = g[case]
    causal = case == "causal"
    o, lse = oracle.attention_head_fwd64(q, k, v, causal, inp["scale"])
    assert np.max(np.abs(o - _arr(c["o"]))) <= 1e-14
    assert np.max(np.abs(lse - np.array([_num(x) for x in c["lse"]]))) <= 1e-14
    dq, dk, dv = oracle.attention_head_bwd64(q, k, v, do, causal, inp["scale"])
    for got, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert np.max(np.abs(got - _arr(c[name]))) <= 1e-14, name
