"""Pins for the fixed-quota rule oracle: hand-worked schedules, brute force, reductions."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import quota as oq
from oracle import step as ostep

GOLD = os.path.join(os.path.dirname(__file__), "golden")
EX = json.load(open(os.path.join(GOLD, "quota_examples.json")))


@pytest.mark.parametrize("ex", EX["schedules"], ids=lambda e: e["name"])
def test_schedule_hand_examples(ex):
    assert oq.quota_schedule(ex["L"], ex["S"]) == ex["quota"]


@pytest.mark.parametrize("ex", EX["remaining"], ids=lambda e: e["name"])
def test_remaining_hand_examples(ex):
    assert oq.quota_for_remaining(ex["L"], ex["S"], ex["masked"]) == ex["quota"]


@pytest.mark.parametrize("ex", EX["topk"], ids=lambda e: e["name"])
def test_topk_hand_examples(ex):
    conf = np.array([-1.0 if c is None else c for c in ex["conf"]])
    assert oq.decide_topk(conf, np.array(ex["mask"], bool), ex["k"]).astype(int).tolist() == ex["unmask"]


@pytest.mark.parametrize("L", [1, 2, 5, 16, 31, 32, 33, 64, 100])
@pytest.mark.parametrize("S", [1, 3, 7, 8, 31, 32, 64, 200])
def test_schedule_sums_to_L_and_is_even(L, S):
    ks = oq.quota_schedule(L, S)
    assert len(ks) == S and sum(ks) == L
    assert max(ks) - min(ks) <= 1
    assert ks == sorted(ks, reverse=True)          # the larger quotas come first


@pytest.mark.parametrize("L,S", [(32, 32), (32, 10), (5, 8), (64, 32), (7, 3), (1, 1)])
def test_following_the_schedule_finishes_in_min_S_L_steps(L, S):
    m, steps = L, 0
    while m > 0:
        k = oq.quota_for_remaining(L, S, m)
        assert k == oq.quota_schedule(L, S)[steps]   # on schedule: the step's own quota
        assert k >= 1
        m -= k
        steps += 1
    assert steps == min(S, L)


def test_topk_brute_force():
    # against exhaustive search: the chosen set maximises the sum of confidences among all sets of
    # size min(k, masked), and among those is lexicographically smallest in slot order
    rng = np.random.default_rng(3)
    for _ in range(300):
        L = int(rng.integers(1, 7))
        masked = rng.random(L) < 0.7
        conf = rng.choice([0.1, 0.2, 0.5, 0.9], L)       # few values: many ties
        k = int(rng.integers(0, L + 2))
        js = [j for j in range(L) if masked[j]]
        n = min(k, len(js))
        best = None
        for comb in itertools.combinations(js, n):
            key = (-sum(conf[j] for j in comb), comb)
            best = key if best is None or key < best else best
        want = np.zeros(L, bool)
        for j in (best[1] if best else ()):
            want[j] = True
        assert np.array_equal(oq.decide_topk(conf, masked, k), want)


def test_quota_one_equals_the_threshold_fallback():
    # k = 1 chooses what the LowConfidence fallback chooses when no slot exceeds the threshold
    rng = np.random.default_rng(4)
    for _ in range(200):
        L = int(rng.integers(1, 40))
        masked = rng.random(L) < 0.6
        if not masked.any():
            continue
        conf = rng.choice([0.05, 0.1, 0.2, 0.3], L)
        assert np.array_equal(oq.decide_topk(conf, masked, 1), ostep.decide(conf, masked, np.float32(0.99)))


def test_step_quota_write_back_and_done():
    # a 2-row box: scores from step.score, k from the schedule, write-back in the last L columns
    L, V, W, S = 4, 6, 7, 2
    rng = np.random.default_rng(5)
    logits = rng.normal(0, 1, (2, L, V)).astype(np.float32)
    ids = np.arange(2 * W, dtype=np.int32).reshape(2, W)
    mask = np.array([[1, 1, 1, 1], [0, 1, 0, 1]], np.uint8)
    out = oq.step_quota(logits, "fp32", ids, mask, S)
    # row 0: block start, schedule (2, 2) -> 2 slots; row 1: 2 masked left = after one step -> 2
    assert out["unmask"][0].sum() == 2 and out["unmask"][1].sum() == 2
    assert out["done"].tolist() == [0, 1] and out["accept"].tolist() == [0, L]
    for r in range(2):
        for j in range(L):
            if out["unmask"][r, j]:
                assert out["ids"][r, W - L + j] == out["argmax"][r, j]
            else:
                assert out["ids"][r, W - L + j] == ids[r, W - L + j]
        assert np.array_equal(out["ids"][r, :W - L], ids[r, :W - L])    # prompt columns untouched
    ref = ostep.step(logits, "fp32", ids, mask, np.array([0.0, 0.0], np.float32))
    assert np.array_equal(out["conf"], ref["conf"]) and np.array_equal(out["argmax"], ref["argmax"])
