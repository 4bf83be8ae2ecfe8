"""Seeded synthetic workloads, five of them (request-level draws only).

Input generation, shared by the GPU path's tests/bench and by the oracle's tests.  Nothing here
computes any part of the unmasking method: it only draws prompt lengths, generation lengths,
block indices, thresholds, masked slots and token ids, and lays them out as a request table.

Citation key for the shapes borrowed from the pages:
  [BlockServe] = page "BlockServe: 块粒度连续批处理实现高吞吐扩散大语言模型服务"
  [DiLaServe]  = page "DiLaServe: High SLO Attainment Serving for Diffusion Language Models"
Block length L = 32 and bf16 logits follow [BlockServe] §III-A; generation length 256 follows the
output length of [DiLaServe] §五 setup; the threshold candidates {0.5,...,0.9} and the default 0.9
follow [DiLaServe] §四 4.1 (paper §3.1).  Vocabulary sizes 126464 / 152064 are those of the
LLaDA / Dream shaped workloads.  Every draw comes from numpy's default_rng(seed) with a fixed seed per
workload (1001 ... 1005).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

QUEUED, ACTIVE, FINISHED = 0, 1, 2
TAU_SET = (0.5, 0.6, 0.7, 0.8, 0.9)


@dataclasses.dataclass
class Workload:
    name: str
    seed_id: int        # fixed per workload: the draws use default_rng(1000 + seed_id)
    L: int
    V: int
    dtype: str          # "fp32" or "bf16"
    sigma: int          # noise sd of the synthetic logits
    umax: int           # planted offset ~ U[0, umax)
    logit_seed: int
    mask_id: int
    pad_id: int
    p: np.ndarray       # int32 [n_req] prompt length
    K: np.ndarray       # int32 [n_req] blocks to generate
    b: np.ndarray       # int32 [n_req] current block index
    state: np.ndarray   # int32 [n_req] QUEUED / ACTIVE / FINISHED
    threshold: np.ndarray  # float32 [n_req]
    arena_off: np.ndarray  # int64 [n_req]
    arena: np.ndarray      # int32 [sum(p + K*L)]  prompt | block 0 | ... | block K-1
    blk_mask: np.ndarray   # uint8 [n_req, L]  current block's mask (1 = masked)
    row_req: np.ndarray    # int32 [rows_cap]; first `rows` entries are the active rows
    rows: int
    queue: np.ndarray      # int32 [n_queued] request ids sorted by (p, id)
    budget: int            # token budget beta; 0 = unbounded
    rows_cap: int
    mode: str              # "single" (one step), "sync" or "fdfo"

    @property
    def n_req(self) -> int:
        return int(self.p.shape[0])

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    def copy(self) -> "Workload":
        return dataclasses.replace(
            self, **{f.name: getattr(self, f.name).copy() for f in dataclasses.fields(self)
                     if isinstance(getattr(self, f.name), np.ndarray)})


def _build(name, seed_id, L, V, dtype, sigma, umax, p, K, b, threshold, active, queue_ids, budget,
           rows_cap, mode, masked_sets, rng):
    n = len(p)
    mask_id, pad_id = V, V + 1
    p = np.asarray(p, np.int32)
    K = np.asarray(K, np.int32)
    b = np.asarray(b, np.int32)
    widths = p.astype(np.int64) + K.astype(np.int64) * L
    arena_off = np.zeros(n, np.int64)
    arena_off[1:] = np.cumsum(widths)[:-1]
    arena = np.full(int(widths.sum()), mask_id, np.int32)
    blk_mask = np.ones((n, L), np.uint8)
    state = np.full(n, QUEUED, np.int32)
    for q in range(n):
        o = int(arena_off[q])
        arena[o:o + p[q]] = rng.integers(0, V, p[q])           # prompt tokens
        done_blocks = int(b[q])
        if done_blocks:                                         # blocks already committed
            arena[o + p[q]:o + p[q] + done_blocks * L] = rng.integers(0, V, done_blocks * L)
        cur = o + p[q] + done_blocks * L
        ms = masked_sets[q]
        if ms is not None:                                      # partly decided current block
            blk_mask[q] = 0
            blk_mask[q, ms] = 1
            toks = rng.integers(0, V, L).astype(np.int32)
            toks[ms] = mask_id
            arena[cur:cur + L] = toks
    for q in active:
        state[q] = ACTIVE
    row_req = np.full(rows_cap, -1, np.int32)
    row_req[:len(active)] = active
    queue = np.array(sorted(queue_ids, key=lambda q: (int(p[q]), int(q))), np.int32)
    return Workload(name=name, seed_id=seed_id, L=L, V=V, dtype=dtype, sigma=sigma, umax=umax,
                    logit_seed=1000 + seed_id, mask_id=mask_id, pad_id=pad_id, p=p, K=K, b=b,
                    state=state, threshold=np.asarray(threshold, np.float32), arena_off=arena_off,
                    arena=arena, blk_mask=blk_mask, row_req=row_req, rows=len(active), queue=queue,
                    budget=int(budget), rows_cap=int(rows_cap), mode=mode)


def tiny_step() -> Workload:
    """Tiny step: 4 requests, L=32, V=1024, fp32, sd 1, offset U[0,12]; p~U[8,32]; K=2, b_i = i mod 2;
    exactly 16 of 32 slots masked (seeded permutation); threshold 0.9."""
    rng = np.random.default_rng(1001)
    n, L, V = 4, 32, 1024
    p = rng.integers(8, 33, n)
    ms = [np.sort(rng.permutation(L)[:L // 2]) for _ in range(n)]
    return _build("tiny-step", 1, L, V, "fp32", 1, 12, p, [2] * n, [i % 2 for i in range(n)],
                  [0.9] * n, list(range(n)), [], 0, n, "single", ms, rng)


def llada_sync() -> Workload:
    """LLaDA-shaped synchronous run: 32 requests, L=32, V=126464, bf16, sd 2, offset U[0,14];
    p~U[64,512]; one block each, fully masked; threshold 0.9; step until every block is done."""
    rng = np.random.default_rng(1002)
    n, L, V = 32, 32, 126464
    p = rng.integers(64, 513, n)
    return _build("llada-sync", 2, L, V, "bf16", 2, 14, p, [1] * n, [0] * n, [0.9] * n,
                  list(range(n)), [], 0, n, "sync", [None] * n, rng)


def dream_step() -> Workload:
    """Dream-shaped step with per-request thresholds: 64 requests, L=32, V=152064, bf16, sd 2,
    offset U[0,14]; p~U[64,512], b=0; threshold uniform over {0.5,...,0.9}; masked fraction
    f~U[0.1,1.0] per block -> max(1, floor(f*L + 0.5)) slots, the first of a seeded permutation."""
    rng = np.random.default_rng(1003)
    n, L, V = 64, 32, 152064
    p = rng.integers(64, 513, n)
    tau = rng.choice(np.array(TAU_SET), n)
    ms = []
    for _ in range(n):
        f = rng.uniform(0.1, 1.0)
        m = max(1, int(math.floor(f * L + 0.5)))
        ms.append(np.sort(rng.permutation(L)[:m]))
    return _build("dream-dynamic-step", 3, L, V, "bf16", 2, 14, p, [1] * n, [0] * n, tau,
                  list(range(n)), [], 0, n, "single", ms, rng)


def blockserve_mixed() -> Workload:
    """BlockServe mixed-state run: 128 active requests with p~U[32,1024], g=256 (K=8), b~U{0..7},
    each at a fresh fully-masked block; 512 more queued with the same p law, sorted by (p, id);
    token budget 262144; threshold 0.9; V=126464 bf16, sd 2, offset U[0,14]; first-done-first-out."""
    rng = np.random.default_rng(1004)
    n_act, n_q, L, V = 128, 512, 32, 126464
    n = n_act + n_q
    p = rng.integers(32, 1025, n)
    b = np.zeros(n, np.int64)
    b[:n_act] = rng.integers(0, 8, n_act)
    return _build("blockserve-mixed", 4, L, V, "bf16", 2, 14, p, [8] * n, b, [0.9] * n,
                  list(range(n_act)), list(range(n_act, n)), 262144, n, "fdfo", [None] * n, rng)


def large_fdfo() -> Workload:
    """Large first-done-first-out run: up to 256 rows, L=64, V=152064 bf16, sd 2, offset U[0,16];
    2048 queued requests, p~U[256,4096], g~U[128,1024] (K = ceil(g/64)), threshold uniform over
    {0.5,...,0.9}; starts empty; no token budget."""
    rng = np.random.default_rng(1005)
    n, L, V = 2048, 64, 152064
    p = rng.integers(256, 4097, n)
    g = rng.integers(128, 1025, n)
    K = (g + L - 1) // L
    tau = rng.choice(np.array(TAU_SET), n)
    return _build("large-fdfo", 5, L, V, "bf16", 2, 16, p, K, [0] * n, tau, [], list(range(n)),
                  0, 256, "fdfo", [None] * n, rng)


WORKLOADS = {"tiny-step": tiny_step, "llada-sync": llada_sync, "dream-dynamic-step": dream_step,
             "blockserve-mixed": blockserve_mixed, "large-fdfo": large_fdfo}
LOOPS = ("llada-sync", "blockserve-mixed", "large-fdfo")   # the workloads that run as whole loops


def make(name: str) -> Workload:
    return WORKLOADS[name]()


def small(L=4, V=64, n_act=3, n_q=5, K=2, seed=7, dtype="fp32", budget=0, rows_cap=None,
          p_range=(1, 9), tau=None, mode="fdfo", sigma=1, umax=8) -> Workload:
    """Small seeded workload of the same structure, for brute-force and loop tests."""
    rng = np.random.default_rng(seed)
    n = n_act + n_q
    p = rng.integers(p_range[0], p_range[1] + 1, n)
    Ks = rng.integers(1, K + 1, n) if K > 1 else np.ones(n, np.int64)
    taus = rng.choice(np.array(TAU_SET), n) if tau is None else np.full(n, tau)
    w = _build("small", 0, L, V, dtype, sigma, umax, p, Ks, [0] * n, taus, list(range(n_act)),
               list(range(n_act, n)), budget, rows_cap or n, mode, [None] * n, rng)
    w.logit_seed = 1000 + seed
    return w
