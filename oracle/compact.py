"""Oracle for block-boundary compaction: scatter, advance/evict, token-budget admission, row layout.

Test infrastructure only (see the package docstring).

From the pages:
  * [FDFO] §FDFO 的核心思想: a request whose current block finishes leaves the batch at once,
    commits its result and frees or reuses its resources; an unfinished request keeps its
    half-finished block and algorithm state for the next round.
  * [FDFO] §工程设计二: per-request result handling — unfinished: store the partial block;
    finished: write the whole block to the output, update the finish state, free at request end.
  * [FDFO] §工程设计四: an unfinished block keeps its request slot in place (no free/alloc churn).
  * [BlockServe] §II-C Algorithm 1: admit from the pending queue under Cost(A ∪ {r_cand}) <= beta,
    run a block cycle, advance b_i, evict requests with b_i >= K_i or an end-of-sequence token.
  * [BlockServe] §II-D: the pending queue is kept sorted by prompt length; refill looks for a
    candidate whose initial width p + L fits the current box without widening it ("sand filling")
    and admits it only if Cost(A ∪ {r_cand}) <= beta (Eq.(1)).
  * [BlockServe] §II-E 向量化混合调度执行: each block starts fully masked; scatter writes the
    denoised block back to its request.
  * [BlockServe] §II-B Figure 1 caption: freed slots are refilled from the sorted queue.

Readings (the pages leave these open):
  * queue order is ascending (p, request id);
  * sand-fill = best fit: the largest p with p + L <= current width, ties to the lowest id; if none
    fits, the smallest p (the least widening); admission stops at the first rejected candidate;
  * Cost <= beta is checked only at admission, with the candidate at block 0;
  * a request whose block finished but has blocks left stays in its row with a fresh, fully
    masked block;
  * rows: admissions take freed rows in ascending order, then new rows at the end; leftover holes
    are filled by moving the highest-index active rows into the lowest holes; survivors otherwise
    keep their row;
  * end-of-sequence (eos_id >= 0) finishes a request whose just-committed block contains eos_id.
"""
from __future__ import annotations

import numpy as np

from .pack import row_width

QUEUED, ACTIVE, FINISHED = 0, 1, 2


class CapacityError(RuntimeError):
    """The queue's candidate cannot be admitted even into an empty batch."""


def choose_candidate(queue_p, taken, W_A: int, L: int):
    """Index (into the sorted queue) of the next candidate, or None if every entry is taken.

    Best fit: among untaken entries with p + L <= W_A, the largest p; the queue is sorted by
    (p, id), so scanning upward with a strict > keeps the lowest id among equal p.  If none fits,
    the first untaken entry (smallest p, lowest id).
    """
    best = None
    for i in range(len(queue_p)):
        if not taken[i] and queue_p[i] + L <= W_A:
            if best is None or queue_p[i] > queue_p[best]:
                best = i
    if best is not None:
        return best
    for i in range(len(queue_p)):
        if not taken[i]:
            return i
    return None


def admit(queue, p, L: int, W_A: int, n_active: int, rows_cap: int, budget: int):
    """Greedy token-budget admission.  Returns (admitted ids in order, new W_A)."""
    queue_p = [int(p[q]) for q in queue]
    taken = [False] * len(queue)
    order = []
    while n_active < rows_cap:
        i = choose_candidate(queue_p, taken, W_A, L)
        if i is None:
            break
        new_W = max(W_A, queue_p[i] + L)
        if budget > 0 and (n_active + 1) * new_W > budget:
            if n_active == 0:
                raise CapacityError(f"request {int(queue[i])} (width {queue_p[i] + L}) exceeds budget {budget}")
            break
        taken[i] = True
        order.append(int(queue[i]))
        n_active += 1
        W_A = new_W
    return order, W_A


def compact(st: dict, rows: int, L: int, W: int, mask_id: int, eos_id: int, budget: int, rows_cap: int,
            box_ids=None, mask=None, done=None):
    """One compaction.  st holds numpy arrays p, K, b, state, threshold, arena_off, arena, blk_mask,
    row_req [rows_cap] and queue; they are updated in place.  With box_ids/mask/done given, the
    box's active blocks are scattered back and finished blocks are committed first; without them
    only admission runs (the start of a run).
    Returns meta dict(rows, W, cost, n_evicted, n_admitted, n_queued)."""
    p, K, b, state = st["p"], st["K"], st["b"], st["state"]
    arena, arena_off, blk_mask, row_req = st["arena"], st["arena_off"], st["blk_mask"], st["row_req"]
    if rows > rows_cap or len(row_req) < rows_cap:
        raise ValueError("rows exceeds rows_cap, or row_req is shorter than rows_cap")

    def block_slice(q, blk):
        start = int(arena_off[q]) + int(p[q]) + int(blk) * L
        return slice(start, start + L)

    freed = []
    n_evicted = 0
    if box_ids is not None:
        # 1. scatter every row's active block (the last L box columns) and mask to its request
        for r in range(rows):
            q = int(row_req[r])
            arena[block_slice(q, b[q])] = box_ids[r, W - L:W]
            blk_mask[q] = mask[r]
        # 2. commit finished blocks: advance, evict or open a fresh fully-masked block
        for r in range(rows):
            if not done[r]:
                continue
            q = int(row_req[r])
            committed = arena[block_slice(q, b[q])]
            b[q] += 1
            hit_eos = eos_id >= 0 and bool(np.any(committed == eos_id))
            if b[q] >= K[q] or hit_eos:
                state[q] = FINISHED
                row_req[r] = -1
                freed.append(r)
                n_evicted += 1
            else:
                arena[block_slice(q, b[q])] = mask_id
                blk_mask[q] = 1

    # 3. admission under the token budget
    survivors = [r for r in range(rows) if row_req[r] >= 0]
    W_A = max((row_width(p[row_req[r]], b[row_req[r]], L) for r in survivors), default=0)
    order, _ = admit(st["queue"], p, L, W_A, len(survivors), rows_cap, budget)
    st["queue"] = np.array([q for q in st["queue"] if int(q) not in set(order)], np.int32)

    # 4. row layout: freed rows ascending, then new rows at the end; then fill holes from the tail
    slots = sorted(freed) + list(range(rows, rows_cap))
    for k, q in enumerate(order):
        r = slots[k]
        row_req[r] = q
        state[q] = ACTIVE
        b[q] = 0
        arena[block_slice(q, 0)] = mask_id
        blk_mask[q] = 1
    n_new = len(survivors) + len(order)
    occupied = [r for r in range(rows_cap) if row_req[r] >= 0]
    holes = [r for r in range(n_new) if row_req[r] < 0]
    movers = sorted([r for r in occupied if r >= n_new], reverse=True)
    assert len(holes) == len(movers)
    for h, t in zip(holes, movers):
        row_req[h] = row_req[t]
        row_req[t] = -1

    # 5. meta
    W_new = max((row_width(p[row_req[r]], b[row_req[r]], L) for r in range(n_new)), default=0)
    return dict(rows=n_new, W=W_new, cost=n_new * W_new, n_evicted=n_evicted, n_admitted=len(order),
                n_queued=int(len(st["queue"])))
