"""Oracle for the host loop rule: synchronous and first-done-first-out (FDFO) execution.

Test infrastructure only (see the package docstring).

From [FDFO] (page "FDFO: 让 dLLM 推理从「整批等最慢」变成「谁先完成谁先走」"):
  * §原来的同步调度问题在哪里: in synchronous mode the batch runs until every block is done; its
    completion time is max_i T_i, and requests that finished earlier wait (the A/B/C example:
    T = 3, 8, 2 wastes (8-3)+(8-8)+(8-2) = 11 request-steps).
  * §工程设计一: _run_sync() repeats forward -> step until all blocks of the batch are done;
    _run_fdfo() runs forward -> step, collects the per-request done flags and yields.
  * §工程设计四: the in-place re-loop — while no block of the batch finishes, keep denoising the
    same batch; as soon as any block finishes, hand control back to the scheduler.
  * §工程设计三: the two modes are an execution switch, orthogonal to the unmasking algorithm.
Reading: admission runs once at the start and after every hand-back to the scheduler
(FDFO: a step with at least one done row; sync: a step with every row done).
A third mode, "handback", is first-done-first-out without the in-place re-loop: control returns to
the scheduler (scatter, admission, re-pack) after every step, which is what §工程设计四 removes by
keeping unfinished blocks in their slots; it produces the same tokens in more scheduler rounds.
"""
from __future__ import annotations

import numpy as np

from .compact import compact
from .pack import pack
from .step import step


def run(st: dict, rows: int, L: int, mask_id: int, pad_id: int, dtype: str, budget: int, rows_cap: int,
        mode: str, logits_fn, eos_id: int = -1, max_steps: int = 1_000_000, max_rounds: int = 0):
    """Drive pack -> (step)* -> compact until the queue and the active set are empty.

    st: request table (see compact()); rows: number of active rows on entry.
    logits_fn(row_req, b_rows, mask_rows) -> logits [rows, L, V] for the current box.
    Returns a trace dict: steps (batch steps), request_steps (rows stepped, summed over steps),
    idle_request_steps (rows stepped with no masked slot left), rounds (hand-backs to the scheduler
    after steps), positions_scored, per-layout metas, and rows (active rows when the run returned).
    max_rounds > 0 stops the run after that many rounds, right after a compact: st and rows are then
    the whole state, and run(st, rows, ...) continues it (its opening admission admits nothing new,
    since the compact just before it stopped admitting on the same state).
    """
    assert mode in ("sync", "fdfo", "handback")
    trace = dict(steps=0, request_steps=0, idle_request_steps=0, rounds=0, positions_scored=0, metas=[], max_cost=0)
    meta = compact(st, rows, L, 0, mask_id, eos_id, budget, rows_cap)
    trace["metas"].append(meta)
    rows, W = meta["rows"], meta["W"]
    while rows > 0:
        trace["max_cost"] = max(trace["max_cost"], meta["cost"])
        pk = pack(st["row_req"], rows, L, W, pad_id, st["p"], st["b"], st["threshold"], st["arena_off"],
                  st["arena"], st["blk_mask"])
        ids, msk = pk["box_ids"], pk["mask"]
        while True:
            if trace["steps"] >= max_steps:
                raise RuntimeError("step limit reached")
            trace["request_steps"] += rows
            trace["idle_request_steps"] += int(np.sum(~(msk != 0).any(axis=1)))
            trace["positions_scored"] += int(np.sum(msk != 0))
            logits = logits_fn(st["row_req"][:rows].copy(), pk["b"], msk)
            out = step(logits, dtype, ids, msk, pk["threshold"], pk["p"], pk["b"])
            ids, msk = out["ids"], out["mask"]
            trace["steps"] += 1
            if mode == "fdfo" and out["done"].any():
                break
            if mode == "sync" and out["done"].all():
                break
            if mode == "handback":
                break
        trace["rounds"] += 1
        meta = compact(st, rows, L, W, mask_id, eos_id, budget, rows_cap, box_ids=ids, mask=msk,
                       done=out["done"])
        trace["metas"].append(meta)
        rows, W = meta["rows"], meta["W"]
        if max_rounds and trace["rounds"] >= max_rounds:
            break
    trace["rows"] = rows
    return trace
