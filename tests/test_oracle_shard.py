"""Pins for the vocabulary-shard oracle: a hand-worked split, and the unsharded result."""
import math

import numpy as np
import pytest

from oracle import shard as osh
from oracle import step as ostep


def test_hand_split_of_the_tie_example():
    # x = (0, 4, 4, 1) in shards (0, 4) | (4, 1): the tie at 4 spans the shards; the lower global
    # index (1) wins; S = (1 + e^-4) + (1 + e^-3) = 2 + e^-3 + e^-4, c = 0.4835349794
    t0 = osh.shard_triple(np.array([0.0, 4.0]), 0)
    t1 = osh.shard_triple(np.array([4.0, 1.0]), 2)
    assert t0 == (4.0, 1, pytest.approx(1 + math.exp(-4)))
    assert t1 == (4.0, 2, pytest.approx(1 + math.exp(-3)))
    m, a, S, c = osh.combine([t0, t1])
    assert (m, a) == (4.0, 1)
    assert S == pytest.approx(2 + math.exp(-3) + math.exp(-4), rel=1e-15)
    assert c == pytest.approx(0.4835349794, abs=1e-10)


def test_split_points():
    assert osh.split_points(10, 3) == [0, 4, 7, 10]
    assert osh.split_points(152064, 8) == [19008 * t for t in range(9)]
    for V in (1, 7, 100, 1001):
        for T in (1, 2, 3, 8):
            if T <= V:
                p = osh.split_points(V, T)
                assert p[0] == 0 and p[-1] == V and all(b > a for a, b in zip(p, p[1:]))


@pytest.mark.parametrize("T", [1, 2, 3, 8])
def test_combine_equals_unsharded(T):
    rng = np.random.default_rng(T)
    for _ in range(50):
        V = int(rng.integers(T, 400))
        x = rng.normal(0, 3, V)
        x[rng.integers(0, V)] += 10
        if rng.random() < 0.3:                         # plant a tie across shard boundaries
            x[rng.integers(0, V)] = x.max()
        pts = osh.split_points(V, T)
        tr = [osh.shard_triple(x[pts[t]:pts[t + 1]], pts[t]) for t in range(T)]
        m, a, S, c = osh.combine(tr)
        m0, a0, S0, c0 = ostep.score(x)
        assert m == m0 and a == a0
        assert S == pytest.approx(S0, rel=1e-13) and c == pytest.approx(c0, rel=1e-13)
