"""Oracle for one denoise step (LowConfidence), float64.

Test infrastructure only (see the package docstring).

What a step computes, from the pages:
  * [FDFO] §工程设计一: the algorithm exposes step(forward_batch, full_logits, states) -> done_flags;
    it reads the logits, updates input_ids by its rule and reports, per block, whether it is done.
  * [FDFO] §工程设计一 (LowConfidence): for every masked slot look at the confidence of the
    predicted token; unmask it if the confidence exceeds the threshold; if no slot in the round
    exceeds it, unmask at least the single most confident slot so the process always advances.
  * [DiLaServe] §三 3.1 (paper §2.1): the confidence is the softmax probability; only slots above
    the preset threshold are unmasked, otherwise the most confident one.  §二 问题定义: each step
    predicts every masked slot in parallel; slots not unmasked stay masked.
  * [FDFO] §工程设计二: the per-request accept length is 0 while the block is unfinished and
    block_size once it can be committed.
  * [DiLaServe] §三 3.2 ①, §四 4.1: thresholds are per request, drawn from a candidate set.
  * [BlockServe] §II-E 逻辑位置对齐: rows are left padded, so every row's active block occupies the
    last L columns of the box.
"""
from __future__ import annotations

import numpy as np


def widen(row, dtype: str) -> np.ndarray:
    """Exact widening of one vocabulary row to float64.

    bf16 rows arrive as uint16 bit patterns: a bfloat16 value is the upper half of a float32,
    so shifting the pattern left by 16 bits gives that float32 exactly; float32 -> float64 is exact.
    """
    if dtype == "bf16":
        return (np.asarray(row, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(row, np.float32).astype(np.float64)


def score(x: np.ndarray):
    """Predicted token and its confidence for one masked slot.

    x: float64 logits over the vocabulary (finite; reading: non-finite logits are a precondition
    violation and are rejected).
    Returns (m, a, S, c) with m = max_v x_v, a = the smallest v with x_v = m (reading: ties go to
    the lowest vocabulary index), S = sum_v exp(x_v - m), and c = 1/S.
    c is the softmax probability of token a:  exp(x_a) / sum_v exp(x_v) = 1 / sum_v exp(x_v - m),
    since x_a = m ([DiLaServe] §三 3.1: softmax probability as the confidence; [FDFO] §工程设计三:
    validated at temperature 0, i.e. the predicted token is the greedy argmax).
    """
    if not np.all(np.isfinite(x)):
        raise ValueError("logits must be finite")
    m = float(np.max(x))
    a = int(np.flatnonzero(x == m)[0])
    S = float(np.sum(np.exp(x - m)))
    return m, a, S, 1.0 / S


def decide(conf: np.ndarray, masked: np.ndarray, tau, return_fallback: bool = False):
    """LowConfidence unmask set for one row's active block.

    conf: float64 [L] confidences (only masked entries are looked at); masked: bool [L];
    tau: the request's threshold as stored (float32), compared in float64.
    Returns bool [L]: U = {masked j : conf_j > tau}; if U is empty while some slot is masked,
    U = {the masked j with the largest conf, lowest j on ties}.  With return_fallback, also
    whether that second case (the fallback) applied.
    Readings: "exceeds" is strict (>); the fallback is per row and unmasks exactly one slot.
    """
    masked = np.asarray(masked, bool)
    t = float(np.float32(tau))
    U = masked & (np.asarray(conf, np.float64) > t)
    fallback = not U.any() and masked.any()
    if fallback:
        best_j, best_c = -1, -np.inf
        for j in range(len(masked)):           # ascending j, strict >: the lowest j wins ties
            if masked[j] and conf[j] > best_c:
                best_j, best_c = j, conf[j]
        U[best_j] = True
    return (U, fallback) if return_fallback else U


def step(logits, dtype: str, input_ids: np.ndarray, mask: np.ndarray, threshold: np.ndarray,
         p=None, b=None, conf_override=None):
    """One denoise step over a packed box.

    logits   : [rows, L, V] (uint16 bf16 patterns or float32); only masked slots are read.
    input_ids: int32 [rows, W] box; the active block of every row is columns W-L .. W-1.
    mask     : uint8 [rows, L], 1 = masked.   threshold: float32 [rows].
    p, b     : optional int [rows]; only used to check that the row fits the box (p+(b+1)L <= W).
    conf_override: optional float64 [rows, L]; when given, the rule is applied to these
    confidences instead of the oracle's own (used to replay a decision taken elsewhere).
    Returns a dict with new ids, mask, done (uint8 [rows]), accept (int32 [rows]), conf (float64
    [rows, L], -1 where not scored), argmax (int64 [rows, L], -1 where not scored), unmask (bool),
    unmasked (int32 [rows]: slots unmasked this step) and fallback (uint8 [rows]: 1 where the row
    had masked slots and none exceeded its threshold, so the single most confident one was taken).
    Reading: a row that enters with no masked slot is left unchanged and reports done=1, accept=L.
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
    unmasked = np.zeros(rows, np.int32)
    fallback = np.zeros(rows, np.uint8)
    for r in range(rows):
        if p is not None and b is not None and int(p[r]) + (int(b[r]) + 1) * L > W:
            raise ValueError(f"row {r} does not fit the box")
        masked = mask[r] != 0
        for j in range(L):
            if masked[j]:
                _, a, _, c = score(widen(logits[r, j], dtype))
                conf[r, j] = c
                arg[r, j] = a
        use = conf[r] if conf_override is None else np.asarray(conf_override[r], np.float64)
        U, fb = decide(use, masked, threshold[r], return_fallback=True)
        unmask[r] = U
        unmasked[r] = int(U.sum())
        fallback[r] = 1 if fb else 0
        for j in range(L):
            if U[j]:
                ids[r, W - L + j] = arg[r, j]
                new_mask[r, j] = 0
        done[r] = 1 if not (new_mask[r] != 0).any() else 0
        accept[r] = L if done[r] else 0
    return dict(ids=ids, mask=new_mask, done=done, accept=accept, conf=conf, argmax=arg, unmask=unmask,
                unmasked=unmasked, fallback=fallback)
