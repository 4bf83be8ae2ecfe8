"""Oracle for vocabulary-sharded scoring: per-shard partial results and their combination, float64.

Test infrastructure only (see the package docstring).

From [DiLaServe] (page "DiLaServe: High SLO Attainment Serving for Diffusion Language Models"):
  * §三 3.2 ② (paper §2.2.2): every denoising step is compute-heavy and tensor parallelism over
    several GPUs cuts its latency; §四 4.5 (paper §3.5): serving runs over tensor-parallel instances.
A tensor-parallel language-model head leaves each GPU with a slice of the vocabulary's logits, so
the step's confidence and predicted token (step.py) must be assembled from per-slice results.

Definition.  For shard t holding columns [o_t, o_t + V_t) of a slot's logits x:
    m_t = max of the slice,  a_t = o_t + (first index of m_t in the slice),  S_t = sum exp(x - m_t).
Combined (shards in ascending order): m = max_t m_t;  a = the smallest a_t with m_t = m;
    S = sum_t S_t * exp(m_t - m);  c = 1 / S.
This is exactly the unsharded result (same max, same first index of the max, the same sum split
into partial sums); only the rounding order of S differs.
"""
from __future__ import annotations

import numpy as np

from .step import score


def shard_triple(x_slice: np.ndarray, offset: int):
    """(m_t, a_t, S_t) of one shard's float64 logits slice, a_t as a global vocabulary index."""
    m, a, S, _ = score(x_slice)
    return m, offset + a, S


def combine(triples):
    """Combine (m_t, a_t, S_t) of shards given in ascending column order -> (m, a, S, c)."""
    m = max(t[0] for t in triples)
    a = min(t[1] for t in triples if t[0] == m)
    S = sum(t[2] * np.exp(t[0] - m) for t in triples)
    return m, a, S, 1.0 / S


def split_points(V: int, T: int) -> list:
    """Column offsets of T contiguous shards of a vocabulary of V (the first V % T one wider)."""
    base, rem = divmod(V, T)
    offs, o = [], 0
    for t in range(T):
        offs.append(o)
        o += base + (1 if t < rem else 0)
    return offs + [V]
