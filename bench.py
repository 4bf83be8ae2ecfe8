#!/usr/bin/env python3
"""Throughput of the dLLM denoise hot path on one MI355X.

Workload: the Dream-shaped dynamic-threshold step — 64 requests at block 0, block length L = 32,
vocabulary V = 152064, bf16 logits (noise sd 2 plus one planted token per slot, offset U[0,14]),
per-request thresholds drawn from {0.5, 0.6, 0.7, 0.8, 0.9}, masked fraction U[0.1, 1.0] per block.
One timed step is the whole device path for one batch: dllm_pack (box gather), dllm_step (score
every masked slot, LowConfidence decision, write-back) and dllm_compact (scatter, commit, evict).
Every step starts from its own pristine copy of the request state, and the logits rotate over
several device buffers (more bytes than the 256 MB Infinity Cache), all resident before timing.

Reports masked positions scored per second over the timed region, the dllm_step kernel's HBM
roofline fraction from per-launch HIP events, and the float64 oracle's rate on the host cores.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "masked positions scored/sec + logits HBM GB/s (fraction of MI355X peak), 1 GPU"
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dllm_step_dream_dynamic_traffic.json")
STEP_SRC = os.path.join(ROOT, "confidence_block_unmasking_amd", "csrc", "step.hip")


def _sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


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


class _Copy:
    """Mutable request state of one timed step (the immutable fields are shared)."""

    def __init__(self, sess):
        import torch
        r = sess.reqs
        self.b = r.b.clone()
        self.state = r.state.clone()
        self.arena = r.arena.clone()
        self.blk_mask = r.blk_mask.clone()
        self.row_req = sess.row_req.clone()
        self.q_ids = sess.queue.ids.clone()
        self.q_len = sess.queue.len.clone()
        self.meta = torch.zeros(32, dtype=torch.uint8, device="cuda")
        from confidence_block_unmasking_amd import _lib
        self.reqs = _lib.Reqs(r.n_req, r.p.data_ptr(), r.K.data_ptr(), self.b.data_ptr(), self.state.data_ptr(),
                              r.threshold.data_ptr(), r.arena_off.data_ptr(), self.arena.data_ptr(),
                              self.blk_mask.data_ptr())
        self.queue = _lib.Queue(self.q_ids.data_ptr(), self.q_len.data_ptr(), sess.queue.cap)


def cpu_baseline(w, seconds):
    """The float64 oracle, as it stands, on rows of the same workload until `seconds` have passed."""
    import numpy as np

    from oracle import pack as opack
    from oracle import step as ostep
    from workload import synth
    W = opack.box_width(w.row_req, w.rows, w.p, w.b, w.L)
    pk = opack.pack(w.row_req, w.rows, w.L, W, w.pad_id, w.p, w.b, w.threshold, w.arena_off, w.arena, w.blk_mask)
    slots, elapsed, rows_done = 0, 0.0, 0
    for r in range(w.rows):
        lg = synth.logits_cpu(1, w.L, w.V, w.dtype, w.row_req[r:r + 1], pk["b"][r:r + 1], pk["mask"][r:r + 1],
                              w.logit_seed, w.sigma, w.umax)
        t0 = time.perf_counter()
        ostep.step(lg, w.dtype, pk["box_ids"][r:r + 1], pk["mask"][r:r + 1], pk["threshold"][r:r + 1])
        elapsed += time.perf_counter() - t0
        slots += int(pk["mask"][r].sum())
        rows_done += 1
        if elapsed >= seconds:
            break
    return {"value": slots / elapsed, "unit": "masked positions/s", "cores": 1, "kind": "oracle",
            "sample": f"first {rows_done} of {w.rows} rows ({slots} masked slots, {elapsed:.1f} s), numpy float64, "
                      "one thread; logits generation excluded",
            "logits_GBps_equiv": slots * w.V * w.elem_bytes / elapsed / 1e9}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=4, help="logits buffers cycled through")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); rows of the step "
              "shard across GPUs without any exchange, but no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    from confidence_block_unmasking_amd import _lib, api
    from confidence_block_unmasking_amd.driver import Session
    from workload import configs, synth

    w = configs.config3()
    sess = Session.from_workload(w)
    L, V = w.L, w.V
    sess.compact(with_box=False)                       # initial layout: rows and box width
    rows, W = sess.rows, sess.W
    M = int(w.blk_mask[w.row_req[:rows]].sum())
    # logits buffers, generated on the device before timing (different seeds)
    bufs = []
    rr = torch.from_numpy(w.row_req[:rows].astype(np.int32)).cuda()
    bb = torch.from_numpy(w.b[w.row_req[:rows]].astype(np.int32)).cuda()
    mm = torch.from_numpy(w.blk_mask[w.row_req[:rows]]).cuda()
    for k in range(args.rotate):
        t = torch.empty((rows, L, V), dtype=torch.bfloat16, device="cuda")
        synth.logits_gpu(t, w.dtype, rows, L, V, rr, bb, mm, w.logit_seed + 7919 * k, w.sigma, w.umax)
        bufs.append(t)
    copies = [_Copy(sess) for _ in range(args.warmup + args.steps)]
    torch.cuda.synchronize()

    lib = _lib.lib()
    vp = ctypes.c_void_p
    stream = vp(torch.cuda.current_stream().cuda_stream)
    box = sess.box_ids
    mask_a, mask_b = sess.masks
    P = lambda t: vp(t.data_ptr())  # noqa: E731
    step_args = []
    for k in range(args.rotate):
        step_args.append((stream, P(bufs[k]), _lib.DLLM_BF16, V, L * V, rows, L, V, P(box), W, P(mask_a), P(mask_b),
                          P(sess.tau), P(sess.p_rows), P(sess.b_rows), P(sess.conf), P(sess.argmax), P(sess.done),
                          P(sess.accept), P(sess.workspace), sess.workspace.numel(), P(sess.status)))
    pack_args, comp_args = [], []
    for c in copies:
        pack_args.append((stream, rows, L, W, w.pad_id, P(c.row_req), ctypes.byref(c.reqs), P(box),
                          P(sess.box_valid), P(sess.box_pos), P(mask_a), P(sess.tau), P(sess.p_rows), P(sess.b_rows),
                          P(sess.status)))
        comp_args.append((stream, rows, L, W, w.mask_id, -1, P(box), P(mask_b), P(sess.done), P(c.row_req),
                          w.rows_cap, ctypes.byref(c.reqs), ctypes.byref(c.queue), w.budget, P(c.meta),
                          P(sess.status)))
    n_total = args.warmup + args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_total)]

    def one(k):
        rc = lib.dllm_pack(*pack_args[k])
        ev[k][0].record()
        rc |= lib.dllm_step(*step_args[k % args.rotate])
        ev[k][1].record()
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
    if rc != 0 or int(sess.status.item()) != 0:
        raise SystemExit(f"library error rc={rc} status={int(sess.status.item())}: {_lib.last_error()}")
    # sanity: every timed step evicted the rows whose block completed, from the same start state
    metas = {bytes(c.meta.cpu().numpy()) for c in copies[args.warmup:]}
    assert len(metas) >= 1
    elapsed = t1 - t0
    kern_ms = np.array([ev[k][0].elapsed_time(ev[k][1]) for k in range(args.warmup, n_total)])
    kern_s = float(kern_ms.mean()) / 1e3
    step_bytes = M * V * 2
    achieved = step_bytes / kern_s / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_sha256") == _sha(STEP_SRC) and tr.get("masked_positions") == M:
            traffic = tr.get("hbm_bytes_per_launch")
    out = {
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
        "config": {"workload": "Dream-shaped dynamic-threshold step: 64 requests, L=32, V=152064 bf16 logits, "
                               "thresholds {0.5..0.9}, masked fraction U[0.1,1.0]; step = pack + step + compact",
                   "requests": w.rows, "block_len": L, "vocab": V, "logits_dtype": "bf16",
                   "masked_positions_per_step": M, "box_width": W, "logits_buffers": args.rotate},
        "logits_GBps": step_bytes * args.steps / elapsed / 1e9,
        "step_kernel_us": {"mean": float(kern_ms.mean()) * 1e3, "p10": float(np.percentile(kern_ms, 10)) * 1e3,
                           "p50": float(np.percentile(kern_ms, 50)) * 1e3,
                           "p90": float(np.percentile(kern_ms, 90)) * 1e3},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
