"""Float64 CPU oracle for the dLLM denoise step, mixed-state packing and FDFO compaction.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import it.  The GPU library never calls it and shares no code with it; the two meet only
through the seeded inputs of the `workload` package.

Every function is the plain definition of what the pages describe, written for a reader to check
by eye, with no blocking, fusion or reordering:

  step.py     confidence/argmax per masked slot, the LowConfidence unmask rule, write-back, done
  pack.py     left-padded bounding-box materialisation with position ids
  compact.py  block-boundary scatter, advance/evict, token-budget admission, row layout
  loop.py     synchronous and first-done-first-out loops, idle request-step accounting
  rows.py     the per-slot confidence/argmax of step.py in C (rows.c), for replaying whole loops
  quota.py, shard.py, features.py   the next rows: fixed per-step quota, vocabulary shards,
              step-predictor features

Citation key (page titles):
  [FDFO]       "FDFO: 让 dLLM 推理从「整批等最慢」变成「谁先完成谁先走」"
  [BlockServe] "BlockServe: 块粒度连续批处理实现高吞吐扩散大语言模型服务"
  [DiLaServe]  "DiLaServe: High SLO Attainment Serving for Diffusion Language Models"
Readings taken where the pages are silent are marked "Reading:" at the point they apply.
Every function here is pinned by tests against hand-worked values, closed forms, library
routines or brute force; none is "parity unpinned".
"""
