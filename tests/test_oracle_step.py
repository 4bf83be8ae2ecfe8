"""Pins for the step oracle: hand-worked examples, closed forms, library routines, invariants."""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import step as ostep

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _bf16(values):
    """float values that are exactly representable in bfloat16 -> uint16 bit patterns."""
    f = np.asarray(values, np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


@pytest.mark.parametrize("ex", _load("scorer_examples.json")["examples"], ids=lambda e: e["name"])
def test_scorer_hand_examples(ex):
    x = np.array(ex["x"], np.float64)
    m, a, S, c = ostep.score(x)
    assert a == ex["argmax"]
    assert m == max(ex["x"])
    assert c == pytest.approx(ex["conf_value"], abs=1e-15)
    assert S == pytest.approx(1.0 / ex["conf_value"], rel=1e-14)


@pytest.mark.parametrize("cf", _load("scorer_examples.json")["closed_forms"], ids=lambda e: e["name"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_scorer_closed_forms_real_vocab(cf, dtype):
    V, d = cf["V"], cf["delta"]
    base = np.full(V, 0.5, np.float32)
    hot = 12345 % V if d else 0
    base[hot] += d
    row = _bf16(base) if dtype == "bf16" else base
    m, a, S, c = ostep.score(ostep.widen(row, dtype))
    assert a == hot
    assert c == pytest.approx(cf["conf_value"], rel=1e-12)
    # the same closed form, derived independently of the stored value
    expect = math.exp(d) / (math.exp(d) + V - 1)
    assert c == pytest.approx(expect, rel=1e-12)


def test_scorer_matches_library_routines():
    rng = np.random.default_rng(0)
    for V in (1, 2, 7, 1024, 126464):
        x = rng.normal(0, 3, V)
        x[rng.integers(0, V)] += rng.uniform(0, 14)
        m, a, S, c = ostep.score(x)
        assert a == int(np.argmax(x))                      # numpy documents first occurrence
        assert c == pytest.approx(math.exp(float(np.max(x)) - logsumexp(x)), rel=1e-12)
        # softmax probability of the predicted token, via scipy
        from scipy.special import softmax
        assert c == pytest.approx(float(softmax(x)[a]), rel=1e-12)


def test_scorer_ties_go_to_lowest_index_and_signed_zero():
    x = np.array([-1.0, 3.0, 2.0, 3.0, 3.0])
    assert ostep.score(x)[1] == 1
    x = np.array([-0.0, 0.0, -1.0])                        # -0.0 == +0.0: lowest index
    assert ostep.score(x)[1] == 0
    assert ostep.score(x)[3] == pytest.approx(1.0 / (2.0 + math.exp(-1.0)))


def test_scorer_rejects_non_finite():
    with pytest.raises(ValueError):
        ostep.score(np.array([0.0, np.nan]))
    with pytest.raises(ValueError):
        ostep.score(np.array([0.0, np.inf]))


def test_scorer_shift_invariance_and_brute_force_tiny():
    # softmax is shift invariant; brute-force the probability definition on tiny rows
    rng = np.random.default_rng(1)
    for _ in range(50):
        V = int(rng.integers(1, 6))
        x = rng.integers(-4, 5, V).astype(np.float64)
        m, a, S, c = ostep.score(x)
        num = math.exp(x[a])
        den = sum(math.exp(v) for v in x)
        assert c == pytest.approx(num / den, rel=1e-13)
        assert all(x[a] > x[v] for v in range(a))         # nothing before a reaches the max
        assert all(x[a] >= v for v in x)
        c2 = ostep.score(x + 7.25)[3]
        assert c2 == pytest.approx(c, rel=1e-13)


def test_widen_bf16_exact():
    vals = np.array([0.0, -0.0, 1.0, -2.5, 3.140625, 1e-3, -65280.0], np.float32)
    u = vals.view(np.uint32)
    u16 = (u >> 16).astype(np.uint16)
    back = ostep.widen(u16, "bf16")
    expect = ((u >> 16) << 16).view(np.float32).astype(np.float64)   # truncation = the bf16 value
    assert np.array_equal(back, expect)
    assert back[2] == 1.0 and back[3] == -2.5 and back[4] == 3.140625


@pytest.mark.parametrize("ex", _load("decision_examples.json")["examples"], ids=lambda e: e["name"])
def test_decision_hand_examples(ex):
    conf = np.array([-1.0 if c is None else c for c in ex["conf"]])
    masked = np.array(ex["mask"], bool)
    U = ostep.decide(conf, masked, np.float32(ex["tau"]))
    assert U.astype(int).tolist() == ex["unmask"]
    U2, fb = ostep.decide(conf, masked, np.float32(ex["tau"]), return_fallback=True)
    assert np.array_equal(U, U2) and int(fb) == ex["fallback"] and int(U.sum()) == ex["unmasked"]
    new_mask = masked & ~U
    assert new_mask.astype(int).tolist() == ex["new_mask"]
    done = int(not new_mask.any())
    assert done == ex["done"]
    assert (len(masked) if done else 0) == ex["accept"]


def test_decision_threshold_compared_as_stored_float32():
    # tau = 0.7 is stored as float32 0.699999988...; a float64 confidence between the two
    # values is above the stored threshold
    tau = np.float32(0.7)
    c = (float(tau) + 0.7) / 2
    assert c > float(tau) and c < 0.7
    U = ostep.decide(np.array([c, 0.1]), np.array([True, True]), tau)
    assert U.tolist() == [True, False]


def _hand_step_case():
    # two rows, L = 4, W = 6 (prompt of 2 in row 0, pad + prompt of 1 in row 1), V = 4
    L, V, W = 4, 4, 6
    logits = np.zeros((2, L, V), np.float32)
    logits[0, 0] = [0, 9, 0, 0]      # conf ~0.9996 -> above 0.9
    logits[0, 1] = [1, 0, 0, 0]      # 1/(1+3/e) ~0.475
    logits[0, 3] = [0, 0, 0, 5]      # ~0.98 -> above
    logits[1, 2] = [2, 2, 0, 0]      # tie between 0 and 1 -> argmax 0, conf ~0.44
    logits[1, 3] = [0, 0, 3, 0]      # ~0.87: below 0.9; largest in the row -> fallback
    ids = np.array([[11, 12, 99, 99, 50, 99], [7, 21, 99, 51, 99, 99]], np.int32)
    mask = np.array([[1, 1, 0, 1], [0, 0, 1, 1]], np.uint8)
    tau = np.array([0.9, 0.9], np.float32)
    return logits, ids, mask, tau, L, W


def test_step_hand_example_full():
    logits, ids, mask, tau, L, W = _hand_step_case()
    out = ostep.step(logits, "fp32", ids, mask, tau)
    assert out["argmax"].tolist() == [[1, 0, -1, 3], [-1, -1, 0, 2]]
    assert out["unmask"].astype(int).tolist() == [[1, 0, 0, 1], [0, 0, 0, 1]]
    assert out["mask"].tolist() == [[0, 1, 0, 0], [0, 0, 1, 0]]
    assert out["ids"].tolist() == [[11, 12, 1, 99, 50, 3], [7, 21, 99, 51, 99, 2]]
    assert out["done"].tolist() == [0, 0]
    assert out["accept"].tolist() == [0, 0]
    assert out["conf"][0, 0] == pytest.approx(math.exp(9) / (math.exp(9) + 3))
    assert out["conf"][1, 3] == pytest.approx(math.exp(3) / (math.exp(3) + 3))
    assert out["conf"][0, 2] == -1.0
    # row 0 unmasks its two slots above 0.9; row 1 has none above, so its fallback takes one
    assert out["unmasked"].tolist() == [2, 1]
    assert out["fallback"].tolist() == [0, 1]


def test_step_invariants_random():
    rng = np.random.default_rng(5)
    for trial in range(20):
        rows, L, V = int(rng.integers(1, 5)), int(rng.integers(1, 9)), int(rng.integers(1, 40))
        W = L + int(rng.integers(0, 6))
        logits = rng.normal(0, 2, (rows, L, V)).astype(np.float32)
        ids = rng.integers(0, 1000, (rows, W)).astype(np.int32)
        mask = (rng.random((rows, L)) < 0.6).astype(np.uint8)
        tau = rng.choice([0.5, 0.6, 0.7, 0.8, 0.9], rows).astype(np.float32)
        out = ostep.step(logits, "fp32", ids, mask, tau)
        for r in range(rows):
            had = mask[r].sum()
            left = out["mask"][r].sum()
            if had:
                assert left < had                              # at least one slot unmasked
            assert np.all(out["mask"][r] <= mask[r])           # mask bits only go 1 -> 0
            assert out["done"][r] == (left == 0)               # done <=> no mask left
            assert out["accept"][r] == (L if left == 0 else 0)
            assert np.array_equal(out["ids"][r, :W - L], ids[r, :W - L])   # prompt untouched
            for j in range(L):
                col = W - L + j
                if mask[r, j] and not out["mask"][r, j]:
                    assert out["ids"][r, col] == np.argmax(logits[r, j])
                else:
                    assert out["ids"][r, col] == ids[r, col]
                if not mask[r, j]:
                    assert out["conf"][r, j] == -1.0 and out["argmax"][r, j] == -1


def test_step_never_reads_unmasked_slots():
    logits, ids, mask, tau, L, W = _hand_step_case()
    poisoned = logits.copy()
    poisoned[mask == 0] = np.nan
    a = ostep.step(logits, "fp32", ids, mask, tau)
    b = ostep.step(poisoned, "fp32", ids, mask, tau)
    for k in ("ids", "mask", "done", "accept", "argmax"):
        assert np.array_equal(a[k], b[k])


def test_step_rejects_row_that_does_not_fit():
    logits, ids, mask, tau, L, W = _hand_step_case()
    with pytest.raises(ValueError):
        ostep.step(logits, "fp32", ids, mask, tau, p=np.array([2, 3]), b=np.array([0, 0]))


def test_steps_per_block_bounded_by_masked_count():
    rng = np.random.default_rng(9)
    L, V, W = 8, 16, 8
    for _ in range(10):
        mask = np.ones((1, L), np.uint8)
        ids = np.zeros((1, W), np.int32)
        tau = np.array([0.9], np.float32)
        n = 0
        while mask.any():
            logits = rng.normal(0, 1, (1, L, V)).astype(np.float32)
            out = ostep.step(logits, "fp32", ids, mask, tau)
            ids, mask = out["ids"], out["mask"]
            n += 1
        assert n <= L
