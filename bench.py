#!/usr/bin/env python3
"""Throughput of the dLLM denoise hot path on one MI355X.

Workload: the Dream-shaped dynamic-threshold step — 64 requests at block 0, block length L = 32,
vocabulary V = 152064, bf16 logits (noise sd 2 plus one planted token per slot, offset U[0,14]),
per-request thresholds drawn from {0.5, 0.6, 0.7, 0.8, 0.9}, masked fraction U[0.1, 1.0] per block.
One timed step is the whole device path for one batch: dllm_pack (box gather), dllm_step_score
(every masked slot's vocabulary row), dllm_step_decide (LowConfidence decision and write-back) and
dllm_compact (scatter, commit, evict).  Every step starts from its own pristine copy of the request
state, and the logits rotate over several device buffers (more bytes than the 256 MB Infinity
Cache), all resident in HBM before timing.

Reports masked positions scored per second over the timed region; the HBM roofline fraction of the
whole dllm_step (scoring kernel start to deciding kernel end) with the scoring kernel's own beside
it, from kernel-bound HIP events on the launch stream over steps run right after the timed region;
and the float64 oracle's rate on the host cores (run first, before the GPU is touched).

Other modes: --step large-fdfo times the same path on the largest single batch (256 requests at
block 0, L=64, V=152064, every slot masked: 4.98 GB of logits per step); --copy-calibration MIB
runs only a plain device copy (for scaling the HBM byte counters); --record-traffic turns
rocprofv3 FETCH_SIZE / WRITE_SIZE runs into the stored traffic figure that later runs report.
"""
import argparse
import ctypes
import glob
import hashlib
import json
import multiprocessing as mp
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "masked positions scored/sec + logits HBM GB/s (fraction of MI355X peak), 1 GPU"
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_kernel_dream_dynamic_traffic.json")
# the scoring kernel's sources (with what they include): the traffic figure is reported only while
# their code, comments and spacing aside, is unchanged
SCORE_SRC = [os.path.join(ROOT, "confidence_block_unmasking_amd", "csrc", f) for f in ("score.hip", "decide.hip",
                                                                                      "step_common.h", "common.h")] + \
            [os.path.join(ROOT, "include", "dllm.h")]
SCORE_KERNEL = "score_kernel"
DECIDE_KERNEL = "decide_kernel<0, 4>"      # the threshold rule at L <= 32
COPY_MIB = 256
SAMPLES = 50          # event-timed steps of each kind after the timed region
DEFAULT_STEP = "dream-dynamic-step"
STEP_WORKLOADS = {
    "dream-dynamic-step": "Dream-shaped dynamic-threshold step: 64 requests, L=32, V=152064 bf16 logits, "
                          "thresholds {0.5..0.9}, masked fraction U[0.1,1.0]; step = pack + score + decide + compact",
    "large-fdfo": "first batch of the large FDFO run: 256 requests admitted at block 0, L=64, V=152064 bf16 "
                  "logits, every slot masked (4.98 GB per step); step = pack + score + decide + compact",
}


def _sha(paths):
    """SHA-256 of the sources' code: comments removed and spacing collapsed, so that editing a comment
    does not void a measurement taken on the same code."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, encoding="utf-8") as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
        h.update(b"\0")
    return h.hexdigest()


# ---- CPU baseline: the float64 oracle as it stands, on host cores ------------------------------

_CPU = {}


def _cpu_worker(args):
    rows_mine, seconds = args
    from oracle import step as ostep
    d = _CPU
    slots, t0 = 0, time.perf_counter()
    while True:
        for r in rows_mine:
            ostep.step(d["logits"][r:r + 1], d["dtype"], d["ids"][r:r + 1], d["mask"][r:r + 1], d["tau"][r:r + 1])
            slots += d["nmask"][r]
            if time.perf_counter() - t0 >= seconds:
                return slots, time.perf_counter() - t0


def _first_batch(w):
    """The workload's first batch as the oracle lays it out: admission by the oracle's compact when
    the workload starts with an empty box, then the oracle's pack.  Returns (row_req, rows, W, pack)."""
    import numpy as np

    from oracle import compact as ocompact
    from oracle import pack as opack
    rows = w.rows
    row_req = w.row_req
    if rows == 0:
        st = dict(p=w.p.astype(np.int64), K=w.K.astype(np.int64), b=w.b.astype(np.int64),
                  state=w.state.astype(np.int64), threshold=w.threshold.copy(), arena_off=w.arena_off.copy(),
                  arena=w.arena.astype(np.int64), blk_mask=w.blk_mask.copy(), row_req=w.row_req.astype(np.int64),
                  queue=w.queue.astype(np.int64))
        m = ocompact.compact(st, 0, w.L, 0, w.mask_id, -1, w.budget, w.rows_cap)
        rows, row_req = m["rows"], st["row_req"]
        p, b, thr, off, arena, blk = st["p"], st["b"], st["threshold"], st["arena_off"], st["arena"], st["blk_mask"]
    else:
        p, b, thr, off, arena, blk = w.p, w.b, w.threshold, w.arena_off, w.arena, w.blk_mask
    W = opack.box_width(row_req, rows, p, b, w.L)
    pk = opack.pack(row_req, rows, w.L, W, w.pad_id, p, b, thr, off, arena, blk)
    return row_req, rows, W, pk


def cpu_baseline(cpu_seconds, name=DEFAULT_STEP, max_logit_bytes=1 << 30):
    """The oracle's step on the first batch of workload `name` (the headline step by default), rows
    spread over a pool of host processes (one thread each), for about `cpu_seconds` of CPU work in
    all.  At most `max_logit_bytes` of logits are generated (the first rows of the batch).  Logits
    generation excluded."""
    from workload import configs, synth
    w = configs.make(name)
    row_req, rows, W, pk = _first_batch(w)
    rows_s = max(1, min(rows, max_logit_bytes // (w.L * w.V * w.elem_bytes)))
    mask = pk["mask"][:rows_s]
    _CPU.update(logits=synth.logits_cpu(rows_s, w.L, w.V, w.dtype, row_req[:rows_s], pk["b"][:rows_s], mask,
                                        w.logit_seed, w.sigma, w.umax),
                dtype=w.dtype, ids=pk["box_ids"][:rows_s], mask=mask, tau=pk["threshold"][:rows_s],
                nmask=[int(x) for x in mask.sum(1)])
    n = max(1, min(16, os.cpu_count() or 1, rows_s))
    per = max(1.0, cpu_seconds / n)
    parts = [list(range(k, rows_s, n)) for k in range(n)]
    os.environ["OMP_NUM_THREADS"] = "1"
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(n) as pool:
        res = pool.map(_cpu_worker, [(rp, per) for rp in parts if rp])
    wall = time.perf_counter() - t0
    slots = sum(s for s, _ in res)
    busy = max(t for _, t in res)
    # the same oracle on one core, over every sampled row in turn
    one_secs = max(1.0, cpu_seconds / 4)
    slots1, busy1 = _cpu_worker((list(range(rows_s)), one_secs))
    _CPU.clear()
    value = slots / busy
    batch = "first batch" if name in configs.LOOPS else "step"
    if rows_s < rows:
        batch += f" ({rows_s} of its {rows} rows)"
    return {"value": value, "unit": "masked positions/s", "cores": len(res), "kind": "oracle",
            "sample": f"{slots} masked-slot scorings of the {batch}, L={w.L}, V={w.V} {w.dtype} (rows round-robin "
                      f"over {len(res)} processes, one thread each, {per:.1f} s each, repeated passes; {wall:.1f} s "
                      "wall); numpy float64; logits generation excluded",
            "logits_GBps_equiv": value * w.V * w.elem_bytes / 1e9,
            "one_core": {"value": slots1 / busy1, "sample": f"{slots1} masked-slot scorings in {busy1:.1f} s, one "
                                                             "process"}}


# ---- HBM byte counters -------------------------------------------------------------------------

def copy_calibration(mib):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)


def _pmc_rows(d):
    """(kernel name, counter, value) rows of a rocprofv3 --pmc run with CSV output under d."""
    import csv
    out = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                out.append((row.get("Kernel_Name", ""), row.get("Counter_Name", ""),
                            float(row.get("Counter_Value", "nan")), row.get("Dispatch_Id", "")))
    if not out:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return out


def _per_dispatch(rows, kernel_pred, counter):
    tot = {}
    for name, cn, v, disp in rows:
        if cn == counter and kernel_pred(name):
            tot[disp] = tot.get(disp, 0.0) + v
    if not tot:
        raise SystemExit(f"no {counter} rows for the kernel")
    vals = sorted(tot.values())
    return vals[len(vals) // 2], len(vals)


def record_traffic(fetch_dir, write_dir, cfetch_dir, cwrite_dir, masked):
    """Median KiB per dispatch of FETCH_SIZE and WRITE_SIZE for the scoring and the deciding kernel,
    each scaled by (known bytes / counted bytes) of a plain copy of COPY_MIB MiB; written to
    TRAFFIC_FILE with their sum, the HBM bytes of one dllm_step."""
    is_copy = lambda n: "copyBuffer" in n or "copy" in n.lower()  # noqa: E731
    known_kib = COPY_MIB * 1024.0
    cf_kib, _ = _per_dispatch(_pmc_rows(cfetch_dir), is_copy, "FETCH_SIZE")
    cw_kib, _ = _per_dispatch(_pmc_rows(cwrite_dir), is_copy, "WRITE_SIZE")
    sf, sw = known_kib / cf_kib, known_kib / cw_kib
    fetch, write = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    rec = {"workload": "Dream-shaped dynamic-threshold step (64 x 32 x 152064 bf16)", "masked_positions": masked,
           "source_sha256": _sha(SCORE_SRC), "copy_mib": COPY_MIB, "copy_fetch_kib": cf_kib, "copy_write_kib": cw_kib,
           "fetch_scale": sf, "write_scale": sw}
    for key, name in (("score_kernel", SCORE_KERNEL), ("decide_kernel", DECIDE_KERNEL)):
        pred = (lambda n, name=name: name in n and "score_kernel<false" not in n and "score_kernel<true, false" not in n)
        f_kib, nf = _per_dispatch(fetch, pred, "FETCH_SIZE")
        w_kib, nw = _per_dispatch(write, pred, "WRITE_SIZE")
        rec[key] = {"kernel": name, "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib,
                    "dispatches": [nf, nw], "hbm_bytes_per_launch": (f_kib * sf + w_kib * sw) * 1024.0}
    rec["hbm_bytes_per_launch"] = rec["score_kernel"]["hbm_bytes_per_launch"]
    rec["dllm_step_hbm_bytes"] = rec["score_kernel"]["hbm_bytes_per_launch"] + rec["decide_kernel"]["hbm_bytes_per_launch"]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec), flush=True)


def stored_traffic(masked):
    """(scoring kernel, whole dllm_step) HBM bytes per launch from TRAFFIC_FILE, or (None, None) when
    the kernels' code changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, None
    with open(TRAFFIC_FILE) as f:
        tr = json.load(f)
    if tr.get("source_sha256") != _sha(SCORE_SRC) or tr.get("masked_positions") != masked:
        return None, None
    return tr.get("hbm_bytes_per_launch"), tr.get("dllm_step_hbm_bytes")


# ---- the timed device path ---------------------------------------------------------------------

class _Copy:
    """Mutable request state of one timed step (the immutable fields are shared)."""

    def __init__(self, sess):
        import torch

        from confidence_block_unmasking_amd import _lib
        r = sess.reqs
        self.b = r.b.clone()
        self.state = r.state.clone()
        self.arena = r.arena.clone()
        self.blk_mask = r.blk_mask.clone()
        self.row_req = sess.row_req.clone()
        self.q_ids = sess.queue.ids.clone()
        self.q_len = sess.queue.len.clone()
        self.meta = torch.zeros(32, dtype=torch.uint8, device="cuda")
        self.reqs = _lib.Reqs(r.n_req, r.p.data_ptr(), r.K.data_ptr(), self.b.data_ptr(), self.state.data_ptr(),
                              r.threshold.data_ptr(), r.arena_off.data_ptr(), self.arena.data_ptr(),
                              self.blk_mask.data_ptr())
        self.queue = _lib.Queue(self.q_ids.data_ptr(), self.q_len.data_ptr(), sess.queue.cap)


def run_gpu(args):
    import numpy as np
    import torch

    from confidence_block_unmasking_amd import _lib, api
    from confidence_block_unmasking_amd.driver import Session
    from workload import configs, synth

    w = configs.make(args.step)
    assert w.dtype == "bf16"
    sess = Session.from_workload(w)
    L, V = w.L, w.V
    sess.compact(with_box=False)                       # initial layout (and admission): rows, box width
    rows, W = sess.rows, sess.W
    h = sess.host_table()
    rq = h["row_req"][:rows].astype(np.int64)
    M = int(h["blk_mask"][rq].sum())
    # logits buffers, generated on the device before timing (different seeds)
    bufs = []
    rr = torch.from_numpy(rq.astype(np.int32)).cuda()
    bb = torch.from_numpy(h["b"][rq].astype(np.int32)).cuda()
    mm = torch.from_numpy(h["blk_mask"][rq]).cuda()
    for k in range(args.rotate):
        t = torch.empty((rows, L, V), dtype=torch.bfloat16, device="cuda")
        synth.logits_gpu(t, w.dtype, rows, L, V, rr, bb, mm, w.logit_seed + 7919 * k, w.sigma, w.umax)
        bufs.append(t)
    n_total = args.warmup + args.steps
    # after the timed steps, a few untimed ones, then 2 * args.samples more of the same kind, each
    # timed by HIP events (the scoring kernel or the whole dllm_step), outside the wall-clock region
    n_settle = 2 * args.rotate          # untimed steps between the timed region and the sampled ones
    n_all = n_total + n_settle + 2 * args.samples
    copies = [_Copy(sess) for _ in range(n_all)]
    torch.cuda.synchronize()

    lib = _lib.lib()
    vp = ctypes.c_void_p
    stream = vp(torch.cuda.current_stream().cuda_stream)
    box = sess.box_ids
    mask_a, mask_b = sess.masks
    P = lambda t: vp(t.data_ptr())  # noqa: E731
    ws, wsn = P(sess.workspace), sess.workspace.numel()
    score_args = [(stream, P(bufs[k]), _lib.DLLM_BF16, V, L * V, rows, L, V, P(mask_a), ws, wsn, P(sess.status))
                  for k in range(args.rotate)]
    if args.rule == "quota":
        decide_fn = lib.dllm_step_decide_quota
        decide_args = (stream, _lib.DLLM_BF16, rows, L, V, P(box), W, P(mask_a), P(mask_b), args.steps_per_block,
                       P(sess.p_rows), P(sess.b_rows), P(sess.conf), P(sess.argmax), P(sess.done), P(sess.accept), ws,
                       wsn, P(sess.status))
    else:
        decide_fn = lib.dllm_step_decide
        decide_args = (stream, _lib.DLLM_BF16, rows, L, V, P(box), W, P(mask_a), P(mask_b), P(sess.tau),
                       P(sess.p_rows), P(sess.b_rows), P(sess.conf), P(sess.argmax), P(sess.done), P(sess.accept), ws,
                       wsn, P(sess.status), None, None)
    if args.shards > 1:
        # vocabulary split into args.shards contiguous slices, scored one after the other (what each
        # rank of a tensor-parallel group would do with its own slice), then combined and decided
        pts = [V * t // args.shards for t in range(args.shards + 1)]
        tri = torch.zeros(rows * L * args.shards * 16, dtype=torch.uint8, device="cuda")
        shard_args = [[(stream, vp(bufs[k].data_ptr() + 2 * pts[t]), _lib.DLLM_BF16, V, L * V, rows, L,
                        pts[t + 1] - pts[t], pts[t], t, args.shards, P(mask_a), ws, wsn, P(tri), P(sess.status))
                       for t in range(args.shards)] for k in range(args.rotate)]
        decide_fn = lib.dllm_step_decide_shards
        decide_args = (stream, args.shards, P(tri), rows, L, V, P(box), W, P(mask_a), P(mask_b),
                       P(sess.tau), P(sess.p_rows), P(sess.b_rows), P(sess.conf), P(sess.argmax), P(sess.done),
                       P(sess.accept), P(sess.status))
    pack_args, comp_args, feat_args = [], [], []
    feats = torch.empty(rows * 9, dtype=torch.float32, device="cuda")
    for c in copies:
        # step-predictor features of the rows after the step (read before compact moves them)
        feat_args.append((stream, rows, L, P(c.row_req), ctypes.byref(c.reqs), P(sess.conf), P(mask_b), P(feats),
                          P(sess.status)))
        pack_args.append((stream, rows, L, W, w.pad_id, P(c.row_req), ctypes.byref(c.reqs), P(box),
                          P(sess.box_valid), P(sess.box_pos), P(mask_a), P(sess.tau), P(sess.p_rows), P(sess.b_rows),
                          P(sess.status)))
        comp_args.append((stream, rows, L, W, w.mask_id, -1, P(box), P(mask_b), P(sess.done), P(c.row_req),
                          w.rows_cap, ctypes.byref(c.reqs), ctypes.byref(c.queue), w.budget, P(c.meta),
                          P(sess.status)))
    # Timing.  The timed region carries no events: each costs the stream some microseconds, which
    # would inflate the step time `value` comes from.  Right after it, on the same state, come
    # 2 * args.samples steps of the same kind, each with one pair of HIP events on the launch stream
    # (torch's current stream), in alternating runs of one step per logits buffer: bound to the
    # scoring kernel's start and end (dllm_step_score_timed), or to the scoring kernel's start and
    # the deciding kernel's end (dllm_step_timed: the whole dllm_step).  So both kinds read every
    # logits buffer.  The vocabulary-shard mode, which has no bound variant, records a pair around the first
    # shard's call instead (that also holds the dispatch latency); the quota rule times only the
    # scoring kernel.
    samp = list(range(n_total + n_settle, n_all))
    # alternate in runs of `rotate` steps, so that both kinds read every logits buffer
    score_k = [k for i, k in enumerate(samp)
               if (i // args.rotate) % 2 == 0 or args.shards > 1 or args.rule != "threshold"]
    step_k = [k for k in samp if k not in score_k]
    kev = {k: api.KernelEvents() for k in score_k} if args.shards <= 1 else {}
    ev = {k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for k in score_k} if args.shards > 1 else {}
    sev = {k: api.KernelEvents() for k in step_k}

    def one(k):
        rc = lib.dllm_pack(*pack_args[k])
        e = ev.get(k)
        if e:
            e[0].record()
        if args.shards > 1:
            sa = shard_args[k % args.rotate]
            rc |= lib.dllm_step_score_shard(*sa[0])
            if e:
                e[1].record()
            for t in range(1, args.shards):
                rc |= lib.dllm_step_score_shard(*sa[t])
        elif k in kev:
            rc |= lib.dllm_step_score_timed(*score_args[k % args.rotate], kev[k].start, kev[k].stop)
        elif k in sev:
            sa = score_args[k % args.rotate]
            rc |= lib.dllm_step_timed(*sa[:8], *decide_args[5:19], sev[k].start, sev[k].stop)
        else:
            rc |= lib.dllm_step_score(*score_args[k % args.rotate])
        if k not in sev:
            rc |= decide_fn(*decide_args)
        if args.features:
            rc |= lib.dllm_step_features(*feat_args[k])
        rc |= lib.dllm_compact(*comp_args[k])
        return rc

    rc = 0
    for k in range(args.warmup):
        rc |= one(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.warmup, n_total):
        rc |= one(k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in range(n_total, n_all):        # a few untimed steps first: the stream is busy again
        rc |= one(k)                       # before the first sampled launch
    torch.cuda.synchronize()
    if rc != 0 or int(sess.status.item()) != 0:
        raise SystemExit(f"library error rc={rc} status={int(sess.status.item())}: {_lib.last_error()}")
    metas = {bytes(c.meta.cpu().numpy()) for c in copies[args.warmup:]}
    if len(metas) != 1:
        raise SystemExit("timed steps from the same start state produced different layouts")
    elapsed = t1 - t0
    # dllm_step (score + decide) from a cold cache, outside the timed region: before each launch a
    # 1 GiB buffer is written, which evicts the logits from L2 and the 256 MB Infinity Cache
    cold_us = None
    if args.cold > 0 and args.shards <= 1:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        kernel_bound = args.rule == "threshold"
        cold_ev = []
        for k in range(args.cold + 2):
            flush.fill_(k & 0xFF)
            if kernel_bound:
                # dllm_step with its events bound to the scoring kernel's start and the deciding
                # kernel's end (the arguments of the two halves, in dllm_step's order)
                e = api.KernelEvents()
                sa, da = score_args[k % args.rotate], decide_args
                rc |= lib.dllm_step_timed(*sa[:8], *da[5:19], e.start, e.stop)
            else:
                e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                e[0].record()
                rc |= lib.dllm_step_score(*score_args[k % args.rotate])
                rc |= decide_fn(*decide_args)
                e[1].record()
            if k >= 2:
                cold_ev.append(e)
        torch.cuda.synchronize()
        if rc != 0:
            raise SystemExit(f"library error rc={rc}: {_lib.last_error()}")
        cms = np.array([e.elapsed_ms() if kernel_bound else e[0].elapsed_time(e[1]) for e in cold_ev]) * 1e3
        med = float(np.median(cms))
        cold_us = {"launches": int(cms.size), "p10": float(np.percentile(cms, 10)), "median": med,
                   "p90": float(np.percentile(cms, 90)),
                   "frac_of_peak_at_median": M * V * 2 / (med * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                   "what": ("dllm_step from the scoring kernel's start to the deciding kernel's end (HIP events "
                            "bound to the two kernels, dllm_step_timed)" if kernel_bound else
                            "dllm_step_score + dllm_step_decide between two HIP events recorded around the calls") +
                           ", each launch after a 1 GiB write that evicts L2 and the Infinity Cache"}
        del flush
    if kev:
        kern_ms = np.array([kev[k].elapsed_ms() for k in score_k])
    else:
        kern_ms = np.array([ev[k][0].elapsed_time(ev[k][1]) for k in score_k])
    by_buf = {}
    for k, t in zip(score_k, kern_ms):
        by_buf.setdefault(k % args.rotate, []).append(float(t) * 1e3)
    step_ms = np.array([sev[k].elapsed_ms() for k in step_k])
    step_bytes = M * V * 2
    timed_bytes = step_bytes if args.shards <= 1 else M * (V // args.shards) * 2

    def dist(ms):
        us = ms * 1e3
        return {"samples": int(us.size), "mean": float(us.mean()), "p10": float(np.percentile(us, 10)),
                "p50": float(np.percentile(us, 50)), "p90": float(np.percentile(us, 90))}
    kern_achieved = timed_bytes / (float(kern_ms.mean()) * 1e-3) / 1e9
    traffic, step_traffic = (stored_traffic(M) if args.shards <= 1 and args.rule == "threshold"
                             and args.step == DEFAULT_STEP else (None, None))
    score_roof = {"kernel": "score_kernel", "achieved": kern_achieved, "frac": kern_achieved / PEAK_HBM_GBPS,
                  "samples": int(kern_ms.size), "traffic": traffic}
    if step_ms.size:
        # the whole dllm_step (scoring kernel, launch boundary, deciding kernel) against the bytes the
        # step must read; the scoring kernel's own fraction beside it
        achieved = step_bytes / (float(step_ms.mean()) * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": "dllm_step (score_kernel start to decide_kernel end)",
                    "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                    "traffic": step_traffic, "samples": int(step_ms.size), "score_kernel": score_roof}
    else:
        roofline = {"bound": "hbm", "kernel": "score_kernel", "achieved": kern_achieved, "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": kern_achieved / PEAK_HBM_GBPS, "traffic": traffic,
                    "samples": int(kern_ms.size)}
    return {
        "metric": METRIC,
        "value": M * args.steps / elapsed,
        "unit": "masked positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": STEP_WORKLOADS[args.step],
                   "rule": "threshold" if args.rule == "threshold" else f"quota, {args.steps_per_block} steps per block",
                   "vocab_shards": max(1, args.shards),
                   **({"features": "dllm_step_features after each decision"} if args.features else {}),
                   "requests": rows, "block_len": L, "vocab": V, "logits_dtype": "bf16",
                   "masked_positions_per_step": M, "box_width": W, "logits_buffers": args.rotate},
        "logits_GBps": step_bytes * args.steps / elapsed / 1e9,
        "score_kernel_us": {**dist(kern_ms),
                            "by_logits_buffer": [round(float(np.mean(by_buf[b])), 2) if b in by_buf else None
                                                 for b in range(args.rotate)],
                            "what": ("HIP events bound to the kernel's start and end (dllm_step_score_timed)"
                                     if kev else "HIP events recorded around the call") +
                                    ", on steps run right after the timed region"},
        **({"dllm_step_us": {**dist(step_ms),
                             "frac_of_peak_at_mean": step_bytes / (float(step_ms.mean()) * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                             "what": "dllm_step (score + decide) from the scoring kernel's start to the deciding "
                                     "kernel's end (dllm_step_timed), on steps run right after the timed region"}}
           if step_ms.size else {}),
        **({"dllm_step_cold_us": cold_us} if cold_us else {}),
        "roofline": roofline,
        **({"timed_kernel": f"dllm_step_score_shard of shard 0 of {args.shards} (scoring + per-slot shard record)"}
           if args.shards > 1 else {}),
    }


# masked-position buckets of the per-step scoring table
M_BUCKETS = (1, 256, 1024, 2048, 4096, 8192, 12288, 16385)


def per_step_table(recs, V, es):
    """recs: (masked positions, rows, scoring-kernel ms, the same logits scored again ms or None) per
    step -> rows of a table by masked-position bucket: steps, mean us, GB/s of each timing."""
    import numpy as np
    out = []
    M = np.array([r[0] for r in recs], np.float64)
    ta = np.array([r[2] for r in recs], np.float64) * 1e-3
    tb = np.array([r[3] if r[3] is not None else np.nan for r in recs], np.float64) * 1e-3
    for lo, hi in zip(M_BUCKETS[:-1], M_BUCKETS[1:]):
        sel = (M >= lo) & (M < hi)
        if not sel.any():
            continue
        by = M[sel].sum() * V * es
        row = {"masked": f"[{lo}, {hi})", "steps": int(sel.sum()), "mean_masked": float(M[sel].mean()),
               "score_us": float(ta[sel].mean() * 1e6), "score_GBps": float(by / ta[sel].sum() / 1e9)}
        if not np.isnan(tb[sel]).all():
            row["rescore_us"] = float(tb[sel].mean() * 1e6)
            row["rescore_GBps"] = float(by / tb[sel].sum() / 1e9)
        out.append(row)
    tot = M.sum() * V * es
    summary = {"steps": len(recs), "score_GBps": float(tot / ta.sum() / 1e9),
               "score_frac": float(tot / ta.sum() / 1e9 / PEAK_HBM_GBPS)}
    if not np.isnan(tb).all():
        summary["rescore_GBps"] = float(tot / tb.sum() / 1e9)
        summary["rescore_frac"] = float(tot / tb.sum() / 1e9 / PEAK_HBM_GBPS)
    return out, summary


def run_loop(name, mode, per_step=False, rescore=False):
    """A whole loop of one workload on the GPU (forward = the synthetic generator on the
    device), with its accounting: batch steps, request-steps, idle request-steps (rows stepped
    after their block finished), scheduler rounds and masked positions scored.  per_step: every
    step's scoring kernel timed by kernel-bound events and tabulated by masked-position count
    (with rescore, the same logits are scored a second time right after, once the forward's
    writes are long finished, and timed the same way)."""
    import torch

    from confidence_block_unmasking_amd import api
    from confidence_block_unmasking_amd.driver import Session
    from workload import configs, synth
    w = configs.make(name)
    mode = mode or w.mode
    if mode == "single":
        raise SystemExit(f"{name} is a single step, not a loop")

    def fwd(sess):
        synth.logits_gpu(sess.logits, w.dtype, sess.rows, w.L, w.V, sess.row_req, sess.b_rows,
                         sess.masks[sess.cur], w.logit_seed, w.sigma, w.umax)
    recs = []

    def timed_step(sess, M):
        # the step as its two halves, the scoring kernel (and its repeat) bound to HIP events
        nxt = 1 - sess.cur
        rows, L, V = sess.rows, sess.L, sess.V
        kw = dict(rows=rows, L=L, V=V, pos_stride=V, row_stride=L * V)
        ea = api.KernelEvents()
        api.dllm_step_score_timed(sess.logits, sess.masks[sess.cur], sess.workspace, sess.status, ea, **kw)
        eb = None
        if rescore:
            eb = api.KernelEvents()
            api.dllm_step_score_timed(sess.logits, sess.masks[sess.cur], sess.workspace, sess.status, eb, **kw)
        api.dllm_step_decide(sess.dtype, rows, L, V, sess.box(), sess.masks[sess.cur], sess.masks[nxt], sess.tau,
                             sess.done, sess.accept, sess.workspace, sess.status, p=sess.p_rows, b=sess.b_rows,
                             conf=sess.conf, argmax=sess.argmax)
        sess.cur = nxt
        recs.append((M, rows, ea, eb))
    # one scheduler round of a throwaway session first, so that every kernel's first launch (code
    # object loading) is outside the timed loop
    warm = Session.from_workload(w)
    warm.run(mode, fwd, max_rounds=1)
    torch.cuda.synchronize()
    del warm
    sess = Session.from_workload(w)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    st = sess.run(mode, fwd, timed=not per_step, step_fn=timed_step if per_step else None)
    torch.cuda.synchronize()
    sec = time.perf_counter() - t0
    if per_step:
        table, summary = per_step_table([(m, r, ea.elapsed_ms(), eb.elapsed_ms() if eb else None)
                                         for m, r, ea, eb in recs], w.V, w.elem_bytes)
        return {"loop": w.name, "mode": mode, "steps": st["steps"], "positions_scored": st["positions_scored"],
                "scoring_by_masked_positions": table, "scoring_overall": summary,
                "what": "scoring kernel per step by kernel-bound HIP events (dllm_step_score_timed)" +
                        ("; rescore: the same logits scored again right after the first scoring" if rescore else "")}
    ph = sess.phase_ms()
    ph["host"] = sec * 1e3 - sum(ph.values())
    keys = ("steps", "request_steps", "idle_request_steps", "rounds", "positions_scored", "evicted", "admitted",
            "max_cost")
    return {"loop": w.name, "mode": mode, "seconds": sec,
            "masked_positions_per_s": st["positions_scored"] / sec, **{k: st[k] for k in keys},
            "phase_ms": ph,
            "step_logits_GBps": st["positions_scored"] * w.V * w.elem_bytes / (ph["step"] / 1e3) / 1e9,
            "note": "wall time includes the synthetic forward (logits generation) of every step; phase_ms sums "
                    "HIP events around every forward, dllm_step, dllm_pack and dllm_compact, and host is the "
                    "rest of the wall time (read-backs of done and mask, scheduling, launches)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--step", choices=tuple(STEP_WORKLOADS), default=DEFAULT_STEP,
                    help="the batch one timed step processes (the default is the headline workload)")
    ap.add_argument("--rotate", type=int, default=4, help="logits buffers cycled through")
    ap.add_argument("--samples", type=int, default=SAMPLES,
                    help="event-timed steps of each kind (scoring kernel, whole dllm_step) after the timed region")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="CPU work of the oracle baseline, in all")
    ap.add_argument("--rule", choices=("threshold", "quota"), default="threshold",
                    help="unmasking rule: LowConfidence threshold (default) or the fixed per-step quota")
    ap.add_argument("--steps-per-block", type=int, default=32, help="diffusion steps per block (quota rule)")
    ap.add_argument("--shards", type=int, default=1, help="score the vocabulary in this many slices and combine")
    ap.add_argument("--cold", type=int, default=100,
                    help="after the timed loop, time this many single dllm_step launches from a flushed cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--features", action="store_true",
                    help="also compute the step-predictor features of every row after each step")
    ap.add_argument("--loop", default=None, metavar="WORKLOAD",
                    help="instead of the step benchmark, run a whole loop: llada-sync, blockserve-mixed or large-fdfo")
    ap.add_argument("--mode", choices=("sync", "fdfo", "handback"), default=None,
                    help="loop mode for --loop (default: the workload's own)")
    ap.add_argument("--per-step", action="store_true",
                    help="with --loop: time every step's scoring kernel and tabulate it by masked positions")
    ap.add_argument("--rescore", action="store_true",
                    help="with --per-step: score each step's logits a second time and time that too")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (HBM counter calibration)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write the traffic file from four rocprofv3 --pmc CSV output folders (no GPU use)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the step runs on one GPU only (asked for --gpus {args.gpus}); its rows would shard "
              "across GPUs without any exchange, but no multi-GPU launcher is provided", file=sys.stderr)
        sys.exit(2)
    if args.samples < 1:
        raise SystemExit("--samples must be at least 1")
    if args.record_traffic:
        from workload import configs
        w = configs.dream_step()
        record_traffic(*args.record_traffic, masked=int(w.blk_mask[w.row_req[:w.rows]].sum()))
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.loop:
        from workload import configs
        if args.loop not in configs.LOOPS:
            raise SystemExit(f"--loop takes one of {', '.join(configs.LOOPS)}")
        if args.per_step:
            print(json.dumps(run_loop(args.loop, args.mode, per_step=True, rescore=args.rescore)), flush=True)
            return
        cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds, args.loop)
        out = run_loop(args.loop, args.mode)
        if cpu is not None:
            cpu["estimated_loop_s"] = out["positions_scored"] / cpu["value"]
            cpu["estimate"] = ("the loop's masked positions scored divided by the sampled rate: the oracle's "
                               "scoring alone, on the same host processes")
            out["cpu_baseline"] = cpu
        print(json.dumps(out), flush=True)
        return
    # the oracle baseline is taken on the headline workload only, before the GPU is touched
    cpu = None if args.no_cpu_baseline or args.step != DEFAULT_STEP else cpu_baseline(args.cpu_seconds, args.step)
    out = run_gpu(args)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
