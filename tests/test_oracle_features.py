"""Pins for the step-predictor feature oracle: hand-worked values and invariants."""
import json
import os

import numpy as np
import pytest

from oracle import features as ofeat

EX = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "feature_examples.json")))


@pytest.mark.parametrize("ex", EX["examples"], ids=lambda e: e["name"])
def test_feature_hand_examples(ex):
    f = ofeat.row_features(np.array(ex["conf"], np.float64), np.array(ex["mask_after"]), np.float32(ex["tau"]),
                           ex["b"], ex["K"], ex["L"])
    want = np.array([np.nan if v is None else v for v in ex["features"]])
    assert np.allclose(f, want, rtol=0, atol=1e-12, equal_nan=True), (f, want)


def test_feature_invariants():
    rng = np.random.default_rng(11)
    for _ in range(500):
        L = int(rng.integers(1, 70))
        K = int(rng.integers(1, 9))
        b = int(rng.integers(0, K))
        scored = rng.random(L) < 0.6
        conf = np.where(scored, rng.random(L), -1.0)
        after = scored & (rng.random(L) < 0.5)
        f = ofeat.row_features(conf, after, np.float32(0.7), b, K, L)
        assert 0.0 <= f[3] <= 1.0 and 0.0 <= f[2] <= 1.0
        assert f[2] * K * L == pytest.approx(b * L + f[3] * L)
        if scored.any():
            c = conf[scored]
            assert f[4] == c.min()
            assert f[4] <= f[5] <= f[6] <= f[8] <= c.max()
            assert c.min() <= f[7] <= c.max()
            n = c.size
            if n % 2 == 1:                                   # odd count: the median is the middle value
                assert f[6] == np.sort(c)[n // 2]
        else:
            assert np.isnan(f[4:]).all()
