"""Pins for the pack and compact oracles: hand-worked examples, brute force, ownership invariants."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import compact as ocompact
from oracle import pack as opack

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _table(reqs, L, K=None, mask_id=-5):
    """Request table from [(p, b, tokens)] with string tokens mapped to ints."""
    n = len(reqs)
    p = np.array([r[0] for r in reqs], np.int64)
    b = np.array([r[1] for r in reqs], np.int64)
    K = np.array(K if K is not None else [r[1] + 1 for r in reqs], np.int64)
    widths = p + K * L
    off = np.zeros(n, np.int64)
    off[1:] = np.cumsum(widths)[:-1]
    arena = np.full(int(widths.sum()), mask_id, np.int64)
    for q, r in enumerate(reqs):
        toks = r[2]
        arena[off[q]:off[q] + len(toks)] = toks
    st = dict(p=p, K=K, b=b, state=np.full(n, 1, np.int64), threshold=np.full(n, 0.9, np.float32),
              arena_off=off, arena=arena, blk_mask=np.ones((n, L), np.uint8),
              row_req=np.arange(n, dtype=np.int64), queue=np.zeros(0, np.int64))
    return st


def test_pack_hand_example_e7():
    g = _load("pack_e7.json")
    L = g["L"]
    names = {}

    def tok(t):
        return names.setdefault(t, len(names) + 100)

    M, P = tok("M"), tok("P")
    reqs = [(r["p"], r["b"], [tok(t) for t in r["tokens"]]) for r in g["requests"]]
    st = _table(reqs, L, mask_id=M)
    W = opack.box_width(st["row_req"], 3, st["p"], st["b"], L)
    assert W == g["W"]
    assert opack.cost(st["row_req"], 3, st["p"], st["b"], L) == g["cost"]
    out = opack.pack(st["row_req"], 3, L, W, P, st["p"], st["b"], st["threshold"], st["arena_off"],
                     st["arena"], st["blk_mask"])
    assert out["box_ids"].tolist() == [[tok(t) for t in row] for row in g["box"]]
    assert out["box_valid"].tolist() == g["valid"]
    assert out["box_pos"].tolist() == g["pos"]
    assert list(range(W - L, W)) == g["active_block_columns"]


def test_pack_invariants_random():
    rng = np.random.default_rng(3)
    for _ in range(30):
        L = int(rng.integers(1, 6))
        n = int(rng.integers(1, 6))
        reqs = []
        for q in range(n):
            p = int(rng.integers(0, 9))
            b = int(rng.integers(0, 3))
            reqs.append((p, b, list(rng.integers(0, 50, p + (b + 1) * L))))
        st = _table(reqs, L)
        st["threshold"] = rng.choice(np.array([0.5, 0.6, 0.7, 0.8, 0.9], np.float32), n)
        st["blk_mask"] = (rng.random((n, L)) < 0.5).astype(np.uint8)
        perm = rng.permutation(n)
        st["row_req"] = perm.astype(np.int64)
        W = opack.box_width(perm, n, st["p"], st["b"], L)
        # brute-force Eq.(1): every width recomputed from scratch
        widths = [reqs[q][0] + (reqs[q][1] + 1) * L for q in perm]
        assert W == max(widths)
        assert opack.cost(perm, n, st["p"], st["b"], L) == n * max(widths)
        extra = int(rng.integers(0, 3))
        out = opack.pack(perm, n, L, W + extra, -1, st["p"], st["b"], st["threshold"], st["arena_off"],
                         st["arena"], st["blk_mask"])
        for r, q in enumerate(perm):
            w = widths[r]
            valid = out["box_valid"][r]
            pos = out["box_pos"][r]
            assert valid.sum() == w and np.all(valid[W + extra - w:] == 1)     # contiguous, right aligned
            assert pos[W + extra - w] == 0                                      # first real token at 0
            assert pos[valid == 1].tolist() == list(range(w))
            assert np.all(pos[valid == 0] == 0)
            assert out["box_ids"][r, valid == 1].tolist() == reqs[q][2]
            assert np.all(out["box_ids"][r, valid == 0] == -1)
            # the per-row views follow the row's request, not the row index
            assert out["threshold"][r] == st["threshold"][q] and out["p"][r] == st["p"][q]
            assert out["b"][r] == st["b"][q] and np.array_equal(out["mask"][r], st["blk_mask"][q])


def test_pack_rejects_too_narrow_box():
    st = _table([(3, 1, [1] * 7)], 2)
    with pytest.raises(ValueError):
        opack.pack(st["row_req"], 1, 2, 6, -1, st["p"], st["b"], st["threshold"], st["arena_off"],
                   st["arena"], st["blk_mask"])


def _e8_state(L, active, queue_p):
    reqs = [(a["p"], a["b"], [7] * (a["p"] + (a["b"] + 1) * L)) for a in active]
    reqs += [(p, 0, [7] * p) for p in queue_p]
    n = len(reqs)
    st = _table(reqs, L, K=[a["b"] + 1 for a in active] + [1] * len(queue_p))
    st["state"][len(active):] = 0
    st["row_req"] = np.concatenate([np.arange(len(active)), np.full(n - len(active), -1)]).astype(np.int64)
    st["queue"] = np.arange(len(active), n, dtype=np.int64)    # queue_p is already ascending
    return st


@pytest.mark.parametrize("case", _load("admission_e8.json")["cases"], ids=lambda c: f"beta{c['beta']}")
def test_admission_hand_example_e8(case):
    g = _load("admission_e8.json")
    L = g["L"]
    st = _e8_state(L, g["active"], g["queue_p"])
    n_req = len(st["p"])
    meta = ocompact.compact(st, 3, L, 0, -5, -1, case["beta"], n_req)
    admitted = [int(st["p"][st["row_req"][r]]) for r in range(3, meta["rows"])]
    assert admitted == case["admitted_p"]
    assert meta["rows"] == case["rows"] and meta["W"] == case["W"] and meta["cost"] == case["cost"]
    assert meta["n_admitted"] == len(case["admitted_p"])


def _brute_choice(queue_p, taken, W_A, L):
    """Every untaken candidate examined: best fit by (p, -index), else the smallest (p, index)."""
    cands = [i for i in range(len(queue_p)) if not taken[i]]
    if not cands:
        return None
    fit = [i for i in cands if queue_p[i] + L <= W_A]
    if fit:
        return max(fit, key=lambda i: (queue_p[i], -i))
    return min(cands, key=lambda i: (queue_p[i], i))


def test_admission_brute_force_tiny():
    rng = np.random.default_rng(11)
    for trial in range(300):
        L = int(rng.integers(1, 4))
        n_act = int(rng.integers(0, 4))
        n_q = int(rng.integers(0, 9))
        act = [dict(p=int(rng.integers(0, 8)), b=int(rng.integers(0, 3))) for _ in range(n_act)]
        qp = sorted(int(x) for x in rng.integers(0, 10, n_q))
        beta = int(rng.integers(0, 60))
        cap = n_act + int(rng.integers(0, 5))
        st = _e8_state(L, act, qp)
        st["row_req"] = np.concatenate([st["row_req"], np.full(max(0, cap - len(st["row_req"])), -1)])
        W_A = max([a["p"] + (a["b"] + 1) * L for a in act], default=0)
        # replay the greedy rule by brute force
        taken = [False] * n_q
        A = [a["p"] + (a["b"] + 1) * L for a in act]
        expect = []
        capacity_error = False
        while len(A) < cap:
            i = _brute_choice(qp, taken, max(A, default=0), L)
            if i is None:
                break
            trial_set = A + [qp[i] + L]
            c = len(trial_set) * max(trial_set)                # Cost recomputed from scratch
            if beta > 0 and c > beta:
                # rejecting the best candidate: every other untaken candidate costs at least as much
                for k in range(n_q):
                    if not taken[k]:
                        s2 = A + [qp[k] + L]
                        assert len(s2) * max(s2) >= c
                capacity_error = len(A) == 0
                break
            taken[i] = True
            expect.append(i)
            A = trial_set
        if capacity_error:
            with pytest.raises(ocompact.CapacityError):
                ocompact.compact(st, n_act, L, 0, -5, -1, beta, cap)
            continue
        meta = ocompact.compact(st, n_act, L, 0, -5, -1, beta, cap)
        got = [int(st["row_req"][r]) - n_act for r in range(n_act, meta["rows"])]
        assert got == expect
        assert meta["W"] == max(A, default=0)
        assert meta["cost"] == len(A) * max(A, default=0)
        if beta > 0 and expect:
            assert meta["cost"] <= beta
        assert meta["n_queued"] == n_q - len(expect)


def _run_random_compacts(seed, steps=40):
    """Random done patterns through compact; returns the history for invariant checks."""
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 4))
    n = int(rng.integers(2, 12))
    reqs = [(int(rng.integers(0, 6)), 0, []) for _ in range(n)]
    K = [int(rng.integers(1, 4)) for _ in range(n)]
    st = _table(reqs, L, K=K, mask_id=-5)
    arena = st["arena"]
    for q in range(n):
        o = st["arena_off"][q]
        arena[o:o + st["p"][q]] = 1000 + q                     # prompt tokens mark their owner
    st["state"][:] = 0
    st["row_req"] = np.full(n, -1, np.int64)
    st["queue"] = np.array(sorted(range(n), key=lambda q: (st["p"][q], q)), np.int64)
    cap = int(rng.integers(1, n + 1))
    beta = int(rng.choice([0, 40, 80]))
    rows, W = 0, 0
    hist = []
    meta = None
    for t in range(steps):
        if t == 0:
            meta = ocompact.compact(st, 0, L, 0, -5, -1, beta, cap)
        else:
            box = np.zeros((rows, W), np.int64)
            for r in range(rows):
                q = st["row_req"][r]
                box[r, W - L:] = 10 * q + st["b"][q]          # the block's "denoised" tokens
            done = (rng.random(rows) < 0.5).astype(np.uint8)
            mask = np.where(done[:, None] == 1, 0, 1).astype(np.uint8) * np.ones((rows, L), np.uint8)
            prev_rows = {int(st["row_req"][r]): r for r in range(rows)}
            meta = ocompact.compact(st, rows, L, W, -5, -1, beta, cap, box_ids=box, mask=mask, done=done)
            hist.append((prev_rows, done))
        rows, W = meta["rows"], meta["W"]
        active = [int(q) for q in st["row_req"][:rows]]
        # ownership invariants
        assert len(set(active)) == len(active)                 # each request in at most one row
        assert all(st["state"][q] == 1 for q in active)        # rows hold active requests
        assert np.all(st["row_req"][rows:] == -1)              # rows are dense
        assert sum(st["state"] == 1) == rows
        assert sum(st["state"] == 0) == len(st["queue"])       # queued + active + finished = total
        for q in range(n):
            o = st["arena_off"][q]
            assert np.all(arena[o:o + st["p"][q]] == 1000 + q)  # prompts untouched
        if rows == 0 and len(st["queue"]) == 0:
            break
    return st, L, n


@pytest.mark.parametrize("seed", range(25))
def test_compact_ownership_and_commit_invariants(seed):
    st, L, n = _run_random_compacts(seed, steps=200)
    for q in range(n):
        if st["state"][q] == 2:
            assert st["b"][q] == st["K"][q]                    # finished exactly at its last block
            o = st["arena_off"][q] + st["p"][q]
            blocks = st["arena"][o:o + st["K"][q] * L].reshape(st["K"][q], L)
            for k in range(st["K"][q]):
                assert np.all(blocks[k] == 10 * q + k)         # every block committed once, unchanged
    if len(st["queue"]) == 0 and not np.any(st["state"] == 1):
        assert np.all(st["state"] == 2)


def test_compact_in_place_reuse_and_hole_filling():
    # rows 0..4 hold requests 0..4 (K = 1 except request 1 which has 2 blocks); rows 1 and 3 done
    L = 2
    reqs = [(1, 0, []), (1, 0, []), (1, 0, []), (1, 0, []), (1, 0, [])]
    st = _table(reqs, L, K=[1, 2, 1, 1, 1], mask_id=-5)
    st["row_req"] = np.arange(5, dtype=np.int64)
    W = 3
    box = np.zeros((5, W), np.int64)
    done = np.array([0, 1, 0, 1, 0], np.uint8)
    mask = np.ones((5, L), np.uint8)
    mask[done == 1] = 0
    o1 = int(st["arena_off"][1])
    st["arena"][o1 + 1 + L:o1 + 1 + 2 * L] = 77                 # stale contents of the next block
    meta = ocompact.compact(st, 5, L, W, -5, -1, 0, 5, box_ids=box, mask=mask, done=done)
    # request 1 advanced to block 1 and keeps row 1; request 3 evicted; row 3 refilled from the tail
    assert meta["rows"] == 4 and meta["n_evicted"] == 1 and meta["W"] == 1 + 2 * L
    assert st["row_req"][:4].tolist() == [0, 1, 2, 4]
    assert st["b"][1] == 1 and st["state"][1] == 1 and st["state"][3] == 2
    assert st["blk_mask"][1].tolist() == [1, 1]
    blk1 = st["arena"][st["arena_off"][1] + 1 + L:st["arena_off"][1] + 1 + 2 * L]
    assert np.all(blk1 == -5)                                   # fresh, fully masked block


def test_admission_opens_block_zero_whatever_the_table_held():
    # an admitted request starts at block 0 with a fully masked block, whatever its b, block-0
    # tokens and block mask held before ([BlockServe] §II-C: admission; §II-E: blocks start masked)
    L = 2
    st = _table([(2, 0, [])], L, K=[3], mask_id=-5)
    st["row_req"] = np.full(2, -1, np.int64)
    st["state"][0] = 0
    st["queue"] = np.array([0], np.int64)
    st["b"][0] = 2
    o = int(st["arena_off"][0])
    st["arena"][o + 2:o + 2 + L] = 77
    st["blk_mask"][0] = 0
    meta = ocompact.compact(st, 0, L, 0, -5, -1, 0, 2)
    assert meta["rows"] == 1 and meta["n_admitted"] == 1 and st["row_req"][0] == 0
    assert st["b"][0] == 0 and st["state"][0] == 1
    assert np.all(st["arena"][o + 2:o + 2 + L] == -5) and st["blk_mask"][0].tolist() == [1, 1]
    assert meta["W"] == 2 + L


def test_compact_eos_evicts_early():
    L = 2
    st = _table([(1, 0, [])], L, K=[3], mask_id=-5)
    box = np.array([[0, 42, 8]], np.int64)
    meta = ocompact.compact(st, 1, L, 3, -5, 42, 0, 1, box_ids=box, mask=np.zeros((1, L), np.uint8),
                            done=np.array([1], np.uint8))
    assert meta["rows"] == 0 and st["state"][0] == 2 and meta["n_evicted"] == 1


def test_compact_capacity_error():
    L = 2
    st = _e8_state(L, [], [10])
    st["row_req"] = np.full(4, -1, np.int64)
    with pytest.raises(ocompact.CapacityError):
        ocompact.compact(st, 0, L, 0, -5, -1, 5, 4)


@pytest.mark.parametrize("case", _load("layout_examples.json")["cases"], ids=lambda c: c["name"])
def test_row_layout_hand_examples(case):
    L = 2
    n = max(case["row_req"] + case["queue"]) + 1
    st = _table([(1, 0, [])] * n, L, K=[1] * n, mask_id=-5)
    st["row_req"] = np.array(case["row_req"] + [-1] * (case["rows_cap"] - case["rows"]), np.int64)
    st["state"][:] = 0
    st["state"][case["row_req"]] = 1
    st["queue"] = np.array(case["queue"], np.int64)
    rows, W = case["rows"], 1 + L
    done = np.array(case["done"], np.uint8)
    box = np.zeros((rows, W), np.int64)
    mask = np.where(done[:, None] == 1, 0, 1).astype(np.uint8) * np.ones((rows, L), np.uint8)
    meta = ocompact.compact(st, rows, L, W, -5, -1, 0, case["rows_cap"], box_ids=box, mask=mask, done=done)
    assert meta["rows"] == case["expect_rows"]
    assert st["row_req"][:meta["rows"]].tolist() == case["expect_row_req"]
    assert np.all(st["row_req"][meta["rows"]:] == -1)
