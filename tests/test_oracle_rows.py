"""Pins for the oracle's C row scorer (oracle/rows.c): hand-worked values, closed forms, library
routines, ties, strides and agreement with step.py's score()."""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import rows as orows
from oracle import step as ostep

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _bf16(values):
    f = np.asarray(values, np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_rows_hand_examples(dtype):
    """E1-E3b of the scorer examples, one row each (every value is exact in both formats)."""
    for ex in _load("scorer_examples.json")["examples"]:
        x = np.array([ex["x"]], np.float32)
        a, c = orows.score_rows(_bf16(x) if dtype == "bf16" else x, dtype)
        assert a[0] == ex["argmax"], ex["name"]
        assert c[0] == pytest.approx(ex["conf_value"], rel=1e-14), ex["name"]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_rows_closed_forms_real_vocab(dtype):
    """Constant row plus one raised entry: c = e^d / (e^d + V - 1), a = the raised index."""
    for cf in _load("scorer_examples.json")["closed_forms"]:
        V, d = cf["V"], cf["delta"]
        base = np.full(V, -1.5, np.float32)
        hot = (7919 * (d + 1)) % V if d else 0
        base[hot] += d
        x = np.stack([base, np.roll(base, 3)])
        a, c = orows.score_rows(_bf16(x) if dtype == "bf16" else x, dtype)
        assert list(a) == [hot, (hot + 3) % V if d else 0], cf["name"]
        expect = math.exp(d) / (math.exp(d) + V - 1)
        assert c == pytest.approx([cf["conf_value"]] * 2, rel=1e-12)
        assert c == pytest.approx([expect] * 2, rel=1e-12)


def test_rows_match_library_routines_and_step_score():
    rng = np.random.default_rng(3)
    for V in (1, 2, 7, 1000, 4099, 126464):
        x = rng.normal(0, 3, (5, V)).astype(np.float32)
        x[np.arange(5), rng.integers(0, V, 5)] += rng.uniform(0, 14, 5).astype(np.float32)
        for dtype in ("fp32", "bf16"):
            xin = x if dtype == "fp32" else (x.view(np.uint32) >> 16).astype(np.uint16)
            a, c = orows.score_rows(xin, dtype)
            for i in range(5):
                xd = ostep.widen(xin[i], dtype)
                assert a[i] == int(np.argmax(xd))                       # numpy: first occurrence
                assert c[i] == pytest.approx(math.exp(float(xd.max()) - logsumexp(xd)), rel=1e-12)
                _, a0, _, c0 = ostep.score(xd)
                assert a[i] == a0 and c[i] == pytest.approx(c0, rel=1e-12)


def test_rows_ties_go_to_the_lowest_index():
    x = np.array([[-1.0, 3.0, 2.0, 3.0, 3.0],
                  [3.0, 3.0, 3.0, 3.0, 3.0],
                  [-0.0, 0.0, -1.0, -2.0, -3.0],
                  [0.0, -0.0, -1.0, -2.0, -3.0],
                  [-5.0, -5.0, -5.0, -5.0, -4.0]], np.float32)
    a, c = orows.score_rows(x, "fp32")
    assert list(a) == [1, 0, 0, 0, 4]
    assert c[1] == pytest.approx(0.2, rel=1e-15)
    assert c[2] == pytest.approx(1.0 / (2.0 + math.exp(-1) + math.exp(-2) + math.exp(-3)), rel=1e-14)


def test_rows_strided_rows_and_threads():
    """Rows taken from a wider buffer (row stride > V) score as the same rows copied out; the
    thread count changes nothing."""
    rng = np.random.default_rng(9)
    big = rng.normal(0, 2, (40, 3000)).astype(np.float32)
    view = big[::3, 100:2600]
    a1, c1 = orows.score_rows(view, "fp32", threads=1)
    a2, c2 = orows.score_rows(np.ascontiguousarray(view), "fp32", threads=3)
    assert np.array_equal(a1, a2) and np.array_equal(c1, c2)
    for i in range(view.shape[0]):
        _, a0, _, c0 = ostep.score(view[i].astype(np.float64))
        assert a1[i] == a0 and c1[i] == pytest.approx(c0, rel=1e-12)


def test_rows_reject_non_finite_and_bad_layouts():
    for bad in (np.nan, np.inf, -np.inf):
        x = np.zeros((3, 8), np.float32)
        x[1, 5] = bad
        with pytest.raises(ValueError, match="non-finite"):
            orows.score_rows(x, "fp32")
    with pytest.raises(ValueError):
        orows.score_rows(np.zeros((2, 8), np.float32), "bf16")
    with pytest.raises(ValueError):
        orows.score_rows(np.zeros((2, 8), np.float32)[:, ::2], "fp32")
    a, c = orows.score_rows(np.zeros((0, 8), np.uint16), "bf16")
    assert a.shape == (0,) and c.shape == (0,)
