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


def test_features_of_a_box_row_by_row():
    """features() over a box: each row takes its own threshold, block index and block count.  The
    rows are the hand-worked L = 4 examples, in an order unlike the file's, so a row that read
    another row's threshold, b or K (or its confidences or mask) would show."""
    four = [e for e in EX["examples"] if e["L"] == 4]
    assert len(four) == 4 and len({(e["tau"], e["b"], e["K"]) for e in four}) == 4
    order = [3, 0, 2, 1]
    rows = [four[i] for i in order]
    conf = np.array([e["conf"] for e in rows], np.float64)
    after = np.array([e["mask_after"] for e in rows], np.uint8)
    tau = np.array([e["tau"] for e in rows], np.float32)
    b = np.array([e["b"] for e in rows], np.int64)
    K = np.array([e["K"] for e in rows], np.int64)
    f = ofeat.features(conf, after, tau, b, K, 4)
    assert f.shape == (4, len(ofeat.NAMES))
    for r, e in enumerate(rows):
        want = np.array([np.nan if v is None else v for v in e["features"]])
        assert np.allclose(f[r], want, rtol=0, atol=1e-12, equal_nan=True), (r, f[r], want)
    assert ofeat.features(np.zeros((0, 4)), np.zeros((0, 4), np.uint8), tau[:0], b[:0], K[:0], 4).shape == (0, 9)
