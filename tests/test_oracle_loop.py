"""Pins for the loop oracle: the A/B/C idle-step example and schedule invariance."""
import json
import os

import numpy as np
import pytest

from oracle import loop as oloop
from workload import configs, synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _abc_state(T, L=8, V=16):
    """Three requests whose blocks need exactly T_i steps: T_i masked slots and logits that never
    clear the threshold (a constant row has confidence 1/V), so each step unmasks one slot."""
    n = len(T)
    p = np.full(n, 2, np.int64)
    K = np.ones(n, np.int64)
    off = np.arange(n, dtype=np.int64) * (2 + L)
    arena = np.full(n * (2 + L), -5, np.int64)
    blk_mask = np.zeros((n, L), np.uint8)
    for q, t in enumerate(T):
        blk_mask[q, :t] = 1
        arena[off[q] + 2 + t:off[q] + 2 + L] = 3            # already decided slots
    st = dict(p=p, K=K, b=np.zeros(n, np.int64), state=np.ones(n, np.int64),
              threshold=np.full(n, 0.9, np.float32), arena_off=off, arena=arena, blk_mask=blk_mask,
              row_req=np.arange(n, dtype=np.int64), queue=np.zeros(0, np.int64))
    return st, L, V


def test_abc_idle_request_steps_sync_vs_fdfo():
    g = json.load(open(os.path.join(GOLD, "abc_idle.json")))
    T = [g["T"]["A"], g["T"]["B"], g["T"]["C"]]

    def const_logits(row_req, b_rows, mask_rows):
        return np.zeros((len(row_req), mask_rows.shape[1], 16), np.float32)

    st, L, V = _abc_state(T)
    tr = oloop.run(st, 3, L, -5, -6, "fp32", 0, 3, "sync", const_logits)
    assert tr["steps"] == g["sync_steps"]
    assert tr["idle_request_steps"] == g["sync_idle_request_steps"]
    assert tr["request_steps"] == g["sync_request_steps"] and tr["rounds"] == g["sync_rounds"]
    st, L, V = _abc_state(T)
    tr = oloop.run(st, 3, L, -5, -6, "fp32", 0, 3, "fdfo", const_logits)
    assert tr["idle_request_steps"] == g["fdfo_idle_request_steps"]
    assert tr["steps"] == max(T)
    assert tr["request_steps"] == g["fdfo_request_steps"] and tr["rounds"] == g["fdfo_rounds"]
    st, L, V = _abc_state(T)
    tr = oloop.run(st, 3, L, -5, -6, "fp32", 0, 3, "handback", const_logits)
    assert tr["idle_request_steps"] == g["handback_idle_request_steps"]
    assert tr["request_steps"] == g["handback_request_steps"] and tr["rounds"] == g["handback_rounds"]
    assert tr["steps"] == max(T)


def _gen(w):
    def fn(row_req, b_rows, mask_rows):
        return synth.logits_cpu(len(row_req), w.L, w.V, w.dtype, row_req, b_rows, mask_rows, w.logit_seed,
                                w.sigma, w.umax)
    return fn


def _state(w):
    return dict(p=w.p.copy(), K=w.K.copy(), b=w.b.copy(), state=w.state.copy(), threshold=w.threshold.copy(),
                arena_off=w.arena_off.copy(), arena=w.arena.copy(), blk_mask=w.blk_mask.copy(),
                row_req=w.row_req.copy(), queue=w.queue.copy())


def _final_tokens(st, w):
    out = []
    for q in range(w.n_req):
        o = int(st["arena_off"][q])
        out.append(st["arena"][o:o + int(w.p[q]) + int(w.K[q]) * w.L].copy())
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_schedule_invariance_bs1_sync_fdfo(seed):
    """Each request's final tokens are the same alone, in a synchronous batch, and under FDFO with
    any row capacity or budget: the logits are keyed by the request's own state."""
    w = configs.small(L=4, V=48, n_act=0, n_q=7, K=3, seed=seed, dtype="bf16", sigma=1, umax=6)
    results = []
    for mode, cap, budget in [("sync", 7, 0), ("fdfo", 7, 0), ("fdfo", 2, 0), ("fdfo", 7, 30), ("sync", 3, 0),
                              ("handback", 7, 0), ("handback", 2, 30)]:
        st = _state(w)
        st["row_req"] = np.full(w.n_req, -1, np.int64)
        tr = oloop.run(st, 0, w.L, w.mask_id, w.pad_id, w.dtype, budget, cap, mode, _gen(w))
        assert np.all(st["state"] == 2)
        results.append(_final_tokens(st, w))
    # bs = 1: each request on its own
    alone = []
    for q in range(w.n_req):
        st = _state(w)
        st["row_req"] = np.full(w.n_req, -1, np.int64)
        st["queue"] = np.array([q], np.int32)
        oloop.run(st, 0, w.L, w.mask_id, w.pad_id, w.dtype, 0, 1, "sync", _gen(w))
        o = int(st["arena_off"][q])
        alone.append(st["arena"][o:o + int(w.p[q]) + int(w.K[q]) * w.L].copy())
    for res in results:
        for q in range(w.n_req):
            assert np.array_equal(res[q], alone[q]), f"request {q} differs"
    for q in range(w.n_req):
        assert not np.any(alone[q] == w.mask_id)            # every block fully generated
        o = int(w.arena_off[q])
        assert np.array_equal(alone[q][:w.p[q]], w.arena[o:o + w.p[q]])   # prompt unchanged


def test_fdfo_never_slower_in_steps_than_sync_for_one_batch():
    w = configs.small(L=4, V=48, n_act=0, n_q=6, K=1, seed=4, dtype="fp32", sigma=1, umax=6)
    steps = {}
    for mode in ("sync", "fdfo"):
        st = _state(w)
        st["row_req"] = np.full(w.n_req, -1, np.int64)
        steps[mode] = oloop.run(st, 0, w.L, w.mask_id, w.pad_id, w.dtype, 0, 6, mode, _gen(w))
    assert steps["fdfo"]["idle_request_steps"] == 0
    assert steps["sync"]["positions_scored"] == steps["fdfo"]["positions_scored"]
    assert steps["sync"]["steps"] == steps["fdfo"]["steps"]
    assert steps["fdfo"]["request_steps"] <= steps["sync"]["request_steps"]


@pytest.mark.parametrize("mode", ["sync", "fdfo", "handback"])
def test_resume_from_tables_continues_identically(mode):
    """The request table, arena, block masks, row map and queue are the whole state between two
    scheduler rounds: a run stopped after k rounds and continued from a copy of that state ends
    with the same tables and the same accounting as a run that never stopped."""
    w = configs.small(L=4, V=48, n_act=0, n_q=7, K=3, seed=5, dtype="bf16", sigma=1, umax=6)
    st = _state(w)
    st["row_req"] = np.full(w.n_req, -1, np.int64)
    full = oloop.run(st, 0, w.L, w.mask_id, w.pad_id, w.dtype, 30, 3, mode, _gen(w))
    keys = ("steps", "request_steps", "idle_request_steps", "rounds", "positions_scored")
    for k in (1, 2, full["rounds"] - 1):
        part = _state(w)
        part["row_req"] = np.full(w.n_req, -1, np.int64)
        first = oloop.run(part, 0, w.L, w.mask_id, w.pad_id, w.dtype, 30, 3, mode, _gen(w), max_rounds=k)
        assert first["rounds"] == k
        saved = {name: np.array(v, copy=True) for name, v in part.items()}
        rest = oloop.run(saved, first["rows"], w.L, w.mask_id, w.pad_id, w.dtype, 30, 3, mode, _gen(w))
        for name in ("arena", "b", "state", "blk_mask", "row_req", "queue"):
            assert np.array_equal(saved[name], st[name]), (k, name)
        for key in keys:
            assert first[key] + rest[key] == full[key], (k, key)
        m0, m1 = rest["metas"][0], first["metas"][-1]
        assert (m0["rows"], m0["W"], m0["n_admitted"], m0["n_evicted"]) == (m1["rows"], m1["W"], 0, 0)
        assert first["metas"] + rest["metas"][1:] == full["metas"]
