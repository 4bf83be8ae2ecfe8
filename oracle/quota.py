"""Oracle for the fixed-quota unmasking rule (the per-step transfer quota), float64.

Test infrastructure only (see the package docstring).

From [BlockServe] (page "BlockServe: 块粒度连续批处理实现高吞吐扩散大语言模型服务"):
  * §II-E 向量化混合调度执行: at the start of every block cycle the per-step transfer quota is
    obtained by spreading the block's masked tokens evenly over the S diffusion steps; since every
    block starts fully masked, the quota does not depend on the block.
  * §III-A: default block length L = 32 with S = 32 denoising steps per block.
The step then unmasks, in every row, that many masked slots: the most confident ones (the
confidence and predicted token are those of the LowConfidence step, see step.py).

Readings (the pages leave these open):
  * "evenly": step t of the block (t = 0 .. S-1) takes floor(L/S) tokens, and the first L mod S
    steps take one more, so the S quotas sum to L;
  * the step index is not stored: it is the step at which the schedule's running total of
    unmasked tokens reaches the block's current unmasked count L - m (m = masked slots left).
    When earlier steps followed the schedule this is exact; otherwise (or past step S) the step
    unmasks every remaining slot once the schedule is exhausted;
  * the quota is capped by the masked slots left; ties in confidence go to the lowest slot j.
"""
from __future__ import annotations

import numpy as np

from .step import score, widen


def quota_schedule(L: int, S: int) -> list:
    """Tokens unmasked at each of the S steps of a block of L tokens."""
    if L < 1 or S < 1:
        raise ValueError("L and S must be positive")
    base, rem = divmod(L, S)
    return [base + (1 if t < rem else 0) for t in range(S)]


def quota_for_remaining(L: int, S: int, m: int) -> int:
    """Quota of the step at which m of the block's L slots are still masked."""
    if m <= 0:
        return 0
    ks = quota_schedule(L, S)
    u = L - m                      # unmasked so far
    t, pre = 0, 0
    while t < S and pre + ks[t] <= u:   # the last step whose running total does not exceed u
        pre += ks[t]
        t += 1
    if t >= S:
        return m
    return min(m, ks[t])


def decide_topk(conf: np.ndarray, masked: np.ndarray, k: int) -> np.ndarray:
    """The k most confident masked slots (all of them if fewer); ties to the lowest j."""
    masked = np.asarray(masked, bool)
    js = [j for j in range(len(masked)) if masked[j]]
    js.sort(key=lambda j: (-float(conf[j]), j))
    U = np.zeros(len(masked), bool)
    for j in js[:max(0, int(k))]:
        U[j] = True
    return U


def step_quota(logits, dtype: str, input_ids: np.ndarray, mask: np.ndarray, S: int, conf_override=None):
    """One denoise step with the fixed per-step quota instead of the threshold rule.

    Same layouts and outputs as step.step (left-padded box, active block in the last L columns);
    row r unmasks quota_for_remaining(L, S, masked count of row r) slots.
    """
    rows, L = mask.shape
    W = input_ids.shape[1]
    ids = input_ids.copy()
    new_mask = mask.copy()
    conf = np.full((rows, L), -1.0)
    arg = np.full((rows, L), -1, np.int64)
    done = np.zeros(rows, np.uint8)
    accept = np.zeros(rows, np.int32)
    unmask = np.zeros((rows, L), bool)
    for r in range(rows):
        masked = mask[r] != 0
        for j in range(L):
            if masked[j]:
                _, a, _, c = score(widen(logits[r, j], dtype))
                conf[r, j] = c
                arg[r, j] = a
        use = conf[r] if conf_override is None else np.asarray(conf_override[r], np.float64)
        U = decide_topk(use, masked, quota_for_remaining(L, S, int(masked.sum())))
        unmask[r] = U
        for j in range(L):
            if U[j]:
                ids[r, W - L + j] = arg[r, j]
                new_mask[r, j] = 0
        done[r] = 1 if not (new_mask[r] != 0).any() else 0
        accept[r] = L if done[r] else 0
    return dict(ids=ids, mask=new_mask, done=done, accept=accept, conf=conf, argmax=arg, unmask=unmask)
