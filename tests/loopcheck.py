"""Deferred float64 checks of every scored slot in long lockstep loops (test infrastructure).

A loop of the large workloads scores millions of vocabulary rows.  To compare every slot that a
step unmasks (and, on chosen steps, every slot it scores) with the oracle, the rows to check are
gathered on the device from the logits buffer the step read, copied into pinned host memory, and
scored by the oracle's C row scorer (oracle/rows.c) in a background thread while the loop goes on.
The logits buffer holds the synthetic generator's output (workload/synth_gpu.hip), which a GPU
test compares bit for bit with the CPU generator; the scoring kernel only reads it.  Each loop
still also checks a few slots per step on rows made by the CPU generator, synchronously.

The loop adopts the GPU's decisions as it goes; the checker confirms them afterwards:
  (i)  argmax equal at every checked slot;
  (ii) |conf_gpu - conf_oracle| <= CONF_TOL at every checked slot;
  (iv) for every row whose masked slots were all checked, the GPU's unmask set equals the rule
       applied to the oracle's confidences, except in ambiguous rows (counted).
(iii), the rule on the GPU's own confidences, is checked in the loop itself, on every row.
finish() raises the first failure with its step, row and slot.
"""
from __future__ import annotations

import os
import queue
import threading
import time

import numpy as np

from oracle import rows as orows
from oracle import step as ostep
from tests.parity import CONF_TOL, ambiguous_row


def host_threads():
    """Scorer threads: the CPUs this process may use, at most 16, less one for the loop itself."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n) - 1)


class DeferredChecker:
    """Collects per-step jobs (host rows + the GPU's results for them) and checks them in order
    on a worker thread."""

    CHUNK_ROWS = 1024          # rows per pinned host block (a few hundred MB at the large vocabularies)

    def __init__(self, dtype: str, V: int, threads: int | None = None, max_inflight_bytes: int = 4 << 30):
        self.dtype, self.V = dtype, int(V)
        self.threads = host_threads() if threads is None else int(threads)
        self.max_inflight = int(max_inflight_bytes)
        self._inflight = 0
        self._cv = threading.Condition()
        self._q: queue.Queue = queue.Queue()
        self.error: str | None = None
        self.stats = dict(slots=0, rows_full=0, ambiguous=0, max_err=0.0, jobs=0, score_s=0.0, elems=0)
        self._t = threading.Thread(target=self._work, name="oracle-checker", daemon=True)
        self._t.start()

    # ---- producer side (the loop's thread) ---------------------------------------------------
    def gather(self, logits, flat_slots):
        """Device rows logits.view(-1, V)[flat_slots] copied into pinned host tensors of at most
        CHUNK_ROWS rows each (waits for the copies).  Returns the list of host tensors."""
        import torch
        n = len(flat_slots)
        if n == 0:
            return []
        nbytes = n * self.V * logits.element_size()
        with self._cv:
            while self._inflight > 0 and self._inflight + nbytes > self.max_inflight and self.error is None:
                self._cv.wait()
            self._inflight += nbytes
        idx = torch.from_numpy(np.asarray(flat_slots, np.int64)).to(logits.device)
        flat = logits.reshape(-1, self.V)
        store = torch.int16 if logits.dtype == torch.bfloat16 else torch.float32
        out = []
        for k in range(0, n, self.CHUNK_ROWS):
            g = flat.index_select(0, idx[k:k + self.CHUNK_ROWS])
            host = torch.empty(tuple(g.shape), dtype=store, pin_memory=logits.is_cuda)
            host.copy_(g.view(store), non_blocking=logits.is_cuda)
            out.append(host)
        if logits.is_cuda:
            torch.cuda.current_stream().synchronize()
        return out

    def submit(self, step: int, host, slots, gpu_arg, gpu_conf, rows_full=()):
        """host: gather()'s list; slots: [(row, j)] in the order of its rows; gpu_arg / gpu_conf: the GPU's results for
        them.  rows_full: [(row, masked [L] bool, tau, gpu unmask set [L] bool)] for rows whose
        masked slots are all among `slots`."""
        if not host:
            return
        self._q.put((step, host, list(slots), np.asarray(gpu_arg), np.asarray(gpu_conf, np.float64), list(rows_full)))

    def finish(self):
        """Wait for every job; raise the first failure."""
        self._q.put(None)
        self._t.join()
        if self.error is not None:
            raise AssertionError(self.error)
        return dict(self.stats)

    # ---- the worker ------------------------------------------------------------------------------
    def _work(self):
        while True:
            job = self._q.get()
            if job is None:
                return
            step, host, slots, g_arg, g_conf, rows_full = job
            try:
                if self.error is None:
                    self._check(step, host, slots, g_arg, g_conf, rows_full)
            except Exception as e:                 # recorded, raised by finish()
                self.error = f"step {step}: {type(e).__name__}: {e}"
            finally:
                nbytes = sum(h.numel() * h.element_size() for h in host)
                job = host = None                  # the pinned blocks go back to torch's cache
                with self._cv:
                    self._inflight -= nbytes
                    self._cv.notify_all()

    def _check(self, step, host, slots, g_arg, g_conf, rows_full):
        t0 = time.perf_counter()
        parts = []
        for h in host:
            x = h.numpy()
            parts.append(orows.score_rows(x.view(np.uint16) if self.dtype == "bf16" else x, self.dtype, self.threads))
        a = np.concatenate([p[0] for p in parts])
        c = np.concatenate([p[1] for p in parts])
        self.stats["score_s"] += time.perf_counter() - t0
        self.stats["elems"] += a.size * self.V
        bad = np.flatnonzero(a != g_arg)
        if bad.size:
            i = int(bad[0])
            raise AssertionError(f"argmax at row {slots[i][0]} slot {slots[i][1]}: gpu {int(g_arg[i])}, "
                                 f"oracle {int(a[i])}")
        err = np.abs(g_conf - c)
        if err.size and err.max() > CONF_TOL:
            i = int(np.argmax(err))
            raise AssertionError(f"conf at row {slots[i][0]} slot {slots[i][1]}: gpu {g_conf[i]}, oracle {c[i]}")
        where = {s: i for i, s in enumerate(slots)}
        for (r, masked, tau, gpu_U) in rows_full:
            L = masked.shape[0]
            o_conf = np.full(L, -1.0)
            for j in np.flatnonzero(masked):
                o_conf[j] = c[where[(r, int(j))]]
            if ambiguous_row(o_conf, masked, tau):
                self.stats["ambiguous"] += 1
                continue
            ref = ostep.decide(o_conf, masked, tau)
            if not np.array_equal(gpu_U, ref):
                raise AssertionError(f"row {r}: unmask set {np.flatnonzero(gpu_U).tolist()} differs from the "
                                     f"oracle's {np.flatnonzero(ref).tolist()}")
        self.stats["slots"] += len(slots)
        self.stats["rows_full"] += len(rows_full)
        self.stats["max_err"] = max(self.stats["max_err"], float(err.max()) if err.size else 0.0)
        self.stats["jobs"] += 1
