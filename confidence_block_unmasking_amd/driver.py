"""Host loop driver: synchronous and first-done-first-out (FDFO) execution over libdllm.

[FDFO] = page "FDFO: 让 dLLM 推理从「整批等最慢」变成「谁先完成谁先走」":
  §工程设计一 — _run_sync() repeats forward -> step until every block of the batch is done;
  _run_fdfo() runs forward -> step and hands the per-request done flags back to the scheduler.
  §工程设计二 — the per-request accept lengths cross to the host (accept_length_per_req_cpu).
  §工程设计四 — in-place re-loop: while no block of the batch finishes, keep denoising the same
  batch; as soon as any finishes, yield to the scheduler.
[BlockServe] = page "BlockServe: 块粒度连续批处理实现高吞吐扩散大语言模型服务", §II-C Algorithm 1:
  admission, a block cycle, advance, evict, repeat until queue and active set are empty.

The driver owns the device buffers and the loop rule only; pack, step and compact run in
libdllm.so.  The model forward is not part of this library: the caller passes `forward`, which
fills the session's logits buffer for the current box (a synthetic generator in tests/bench).
Per step the only device-to-host traffic is the done flags and the new mask of the box rows.
"""
from __future__ import annotations

import numpy as np
import torch

from . import api


def _around(events, fn):
    """fn() between the two timing events (if any) on the current stream; the caller's forward is
    timed this way, its own host work included."""
    if events is None:
        return fn()
    events[0].record()
    out = fn()
    events[1].record()
    return out


class Session:
    """Device state for one run: request table, queue, row map, box buffers and step workspace."""

    def __init__(self, p, K, b, state, threshold, arena_off, arena, blk_mask, row_req, rows, queue, *, L, V,
                 dtype=torch.bfloat16, rows_cap, budget=0, mask_id, pad_id, eos_id=-1, device="cuda",
                 logits=None):
        self.L, self.V, self.dtype = int(L), int(V), dtype
        self.rows_cap, self.budget = int(rows_cap), int(budget)
        self.mask_id, self.pad_id, self.eos_id = int(mask_id), int(pad_id), int(eos_id)
        self.device = device
        self.reqs = api.ReqTable(p, K, b, state, threshold, arena_off, arena, blk_mask, device=device)
        self.queue = api.DevQueue(queue, device=device, cap=max(len(queue), 1))
        rr = np.full(self.rows_cap, -1, np.int32)
        rr[:rows] = np.asarray(row_req)[:rows]
        self.row_req = torch.as_tensor(rr).to(device)
        self.rows = int(rows)
        p64 = np.asarray(p, np.int64)
        K64 = np.asarray(K, np.int64)
        self.W_max = int((p64 + K64 * self.L).max()) if len(p64) else self.L
        n = self.rows_cap
        i32, u8, f32 = torch.int32, torch.uint8, torch.float32
        self.box_ids = torch.empty(n * self.W_max, dtype=i32, device=device)
        self.box_valid = torch.empty(n * self.W_max, dtype=u8, device=device)
        self.box_pos = torch.empty(n * self.W_max, dtype=i32, device=device)
        self.masks = [torch.zeros(n * self.L, dtype=u8, device=device) for _ in range(2)]
        self.cur = 0
        self.tau = torch.empty(n, dtype=f32, device=device)
        self.p_rows = torch.empty(n, dtype=i32, device=device)
        self.b_rows = torch.empty(n, dtype=i32, device=device)
        self.done = torch.zeros(n, dtype=u8, device=device)
        self.accept = torch.zeros(n, dtype=i32, device=device)
        self.conf = torch.empty(n * self.L, dtype=f32, device=device)
        self.argmax = torch.empty(n * self.L, dtype=i32, device=device)
        self.workspace = api.new_workspace(n, self.L, self.V, dtype, device=device)
        self.status = torch.zeros(1, dtype=i32, device=device)
        self.meta = torch.zeros(32, dtype=u8, device=device)
        self.features_buf = torch.empty(n * api.N_FEATURES, dtype=f32, device=device)
        # per-row report of the last step (metrics runs): slots unmasked, single-slot fallback taken
        self.unmasked_rows = torch.zeros(n, dtype=i32, device=device)
        self.fallback_rows = torch.zeros(n, dtype=u8, device=device)
        # pinned host copies for the per-step read-back (done, new mask and status in one sync)
        pin = str(device).startswith("cuda")
        self._h_done = torch.empty(n, dtype=u8, pin_memory=pin)
        self._h_mask = torch.empty(n * self.L, dtype=u8, pin_memory=pin)
        self._h_status = torch.empty(1, dtype=i32, pin_memory=pin)
        self.logits = logits if logits is not None else torch.empty((n, self.L, self.V), dtype=dtype, device=device)
        self.W = 0
        self.stats = dict(steps=0, request_steps=0, positions_scored=0, compacts=0, packs=0, rounds=0,
                          idle_request_steps=0, max_cost=0, evicted=0, admitted=0, unmasked=0,
                          fallback_row_steps=0, block_steps={})
        # (start, end) events around each library call and each forward, when a run is timed
        self.events = {"forward": [], "step": [], "pack": [], "compact": []}

    @classmethod
    def from_workload(cls, w, device="cuda", logits=None, eos_id=-1):
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        return cls(w.p, w.K, w.b, w.state, w.threshold, w.arena_off, w.arena, w.blk_mask, w.row_req, w.rows,
                   w.queue, L=w.L, V=w.V, dtype=dt, rows_cap=w.rows_cap, budget=w.budget, mask_id=w.mask_id,
                   pad_id=w.pad_id, eos_id=eos_id, device=device, logits=logits)

    # ---- views of the current box -------------------------------------------------------------
    def box(self):
        return self.box_ids[:self.rows * self.W].view(self.rows, self.W)

    def mask(self):
        return self.masks[self.cur][:self.rows * self.L].view(self.rows, self.L)

    def _readback(self):
        """done [rows] and the current mask [rows, L] on the host, and the status word: three
        asynchronous copies into pinned memory and one synchronisation."""
        n, nl = self.rows, self.rows * self.L
        self._h_done[:n].copy_(self.done[:n], non_blocking=True)
        self._h_mask[:nl].copy_(self.masks[self.cur][:nl], non_blocking=True)
        self._h_status.copy_(self.status, non_blocking=True)
        torch.cuda.current_stream().synchronize()
        return (self._h_done[:n].numpy().copy(), self._h_mask[:nl].numpy().reshape(n, self.L).copy(),
                int(self._h_status[0]))

    def check_status(self, where):
        s = int(self.status.item())
        if s != 0:
            raise api.DllmError(s, where, "(device status)")

    def _timed(self, phase, timed, fn):
        """fn(events): when timed, `events` is a pair of timing events that fn records on the current
        stream right around the work it enqueues (the library calls record them after marshalling
        their arguments, so the interval holds no host work); otherwise None."""
        if not timed:
            return fn(None)
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        out = fn(ev)
        self.events[phase].append(ev)
        return out

    def phase_ms(self):
        """Total milliseconds of each timed phase so far (synchronises)."""
        torch.cuda.synchronize()
        return {k: float(sum(a.elapsed_time(b) for a, b in v)) for k, v in self.events.items()}

    # ---- the three library calls ----------------------------------------------------------------
    def compact(self, with_box=True, timed=False):
        kw = {}
        if with_box and self.rows > 0:
            kw = dict(box_ids=self.box_ids, mask=self.masks[self.cur], done=self.done)
        self._timed("compact", timed, lambda ev: api.dllm_compact(
            self.rows, self.L, self.W, self.mask_id, self.eos_id, self.row_req, self.rows_cap, self.reqs,
            self.queue, self.budget, self.meta, self.status, events=ev, **kw))
        m = api.read_meta(self.meta)
        self.check_status("dllm_compact")
        self.rows, self.W = m["rows"], m["W"]
        self.stats["compacts"] += 1
        self.stats["evicted"] += m["n_evicted"]
        self.stats["admitted"] += m["n_admitted"]
        self.stats["max_cost"] = max(self.stats["max_cost"], m["cost"])
        return m

    def pack(self, timed=False):
        self._timed("pack", timed, lambda ev: api.dllm_pack(
            self.rows, self.L, self.W, self.pad_id, self.row_req, self.reqs, self.box_ids, self.masks[self.cur],
            self.tau, self.p_rows, self.b_rows, self.status, box_valid=self.box_valid, box_pos=self.box_pos,
            events=ev))
        self.stats["packs"] += 1

    def step(self, timed=False, report=False):
        """One dllm_step on the current box.  report=True runs it as its two halves, the deciding one
        also writing each row's count of unmasked slots and fallback flag (unmasked_rows,
        fallback_rows); the results are the same bit for bit."""
        nxt = 1 - self.cur
        if report:
            def both(ev):
                api.dllm_step_score(self.logits, self.masks[self.cur], self.workspace, self.status, rows=self.rows,
                                    L=self.L, V=self.V, pos_stride=self.V, row_stride=self.L * self.V)
                api.dllm_step_decide(self.dtype, self.rows, self.L, self.V, self.box(), self.masks[self.cur],
                                     self.masks[nxt], self.tau, self.done, self.accept, self.workspace, self.status,
                                     p=self.p_rows, b=self.b_rows, conf=self.conf, argmax=self.argmax,
                                     unmasked=self.unmasked_rows, fallback=self.fallback_rows)
            self._timed("step", timed, lambda ev: _around(ev, lambda: both(ev)))
        else:
            self._timed("step", timed, lambda ev: api.dllm_step(
                self.logits, self.box(), self.masks[self.cur], self.masks[nxt], self.tau, self.done, self.accept,
                self.workspace, self.status, p=self.p_rows, b=self.b_rows, conf=self.conf, argmax=self.argmax,
                rows=self.rows, L=self.L, V=self.V, pos_stride=self.V, row_stride=self.L * self.V, events=ev))
        self.cur = nxt

    def features(self):
        """Step-predictor features of the current rows after the last step: device [rows, 9]."""
        api.dllm_step_features(self.rows, self.L, self.row_req, self.reqs, self.conf, self.masks[self.cur],
                               self.features_buf, self.status)
        return self.features_buf[:self.rows * api.N_FEATURES].view(self.rows, api.N_FEATURES)

    # ---- the loop rule ----------------------------------------------------------------------------
    def run(self, mode, forward, max_steps=10**7, on_step=None, timed=False, max_rounds=0, metrics=False,
            step_fn=None):
        """Drive compact -> pack -> (forward, step)* -> compact ... until queue and rows are empty.

        mode: "sync" (the batch runs until every block is done), "fdfo" (first-done-first-out with
        the in-place re-loop: the batch is re-stepped as it stands until some block finishes) or
        "handback" (first-done-first-out that hands control back to the scheduler after every step,
        the behaviour the in-place re-loop removes).  forward(session) fills session.logits for the
        current box.  on_step(session, info) is called after every step with the host copies (done,
        new mask) — the test harness uses it to check each step.  timed: bracket every forward,
        step, pack and compact with events (totals from phase_ms()).  max_rounds > 0 returns after
        that many scheduler rounds, right after a compact, where snapshot() holds the whole state.
        The stats always count the tokens unmasked; metrics=True also reads back the step's per-row
        fallback flags (dllm_step_decide's report: no masked confidence above the threshold) and the
        row map, to count the fallback row-steps and the steps each finished block took
        (stats["block_steps"]: steps -> blocks).  step_fn(session, masked_positions), when given,
        enqueues each step in place of step() (it must leave the new mask in the other mask buffer
        and switch to it, as step() does); measurement code uses it to time the kernels one by one.
        Returns self.stats."""
        assert mode in ("sync", "fdfo", "handback")
        self.compact(with_box=False, timed=timed)    # admission at the start of the run
        in_block = {}                                # request -> steps of its current block
        while self.rows > 0:
            self.pack(timed=timed)
            mask_host = self.mask().cpu().numpy()
            if metrics:
                req_host = self.row_req[:self.rows].cpu().numpy()
            while True:
                if self.stats["steps"] >= max_steps:
                    raise RuntimeError("step limit reached")
                masked = mask_host != 0
                masked_rows = masked.any(axis=1)
                self.stats["request_steps"] += self.rows
                self.stats["idle_request_steps"] += int((~masked_rows).sum())
                self.stats["positions_scored"] += int(masked.sum())
                self._timed("forward", timed, lambda ev: _around(ev, lambda: forward(self)))
                if step_fn is not None:
                    step_fn(self, int(masked.sum()))
                else:
                    self.step(timed=timed, report=metrics)
                done, mask_host, st = self._readback()
                if st != 0:
                    raise api.DllmError(st, "dllm_step", "(device status)")
                self.stats["steps"] += 1
                unmasked = int(masked.sum()) - int((mask_host != 0).sum())
                self.stats["unmasked"] += unmasked
                if metrics:
                    self.stats["fallback_row_steps"] += int(self.fallback_rows[:self.rows].sum().item())
                    for r in np.flatnonzero(masked_rows):
                        q = int(req_host[r])
                        in_block[q] = in_block.get(q, 0) + 1
                        if done[r]:
                            hist = self.stats["block_steps"]
                            hist[in_block[q]] = hist.get(in_block[q], 0) + 1
                            in_block[q] = 0
                if on_step is not None:
                    on_step(self, dict(done=done, mask=mask_host, unmasked=unmasked))
                if mode == "fdfo" and done.any():
                    break
                if mode == "sync" and done.all():
                    break
                if mode == "handback":
                    break
            self.stats["rounds"] += 1
            self.compact(with_box=True, timed=timed)
            if max_rounds and self.stats["rounds"] >= max_rounds:
                break
        return self.stats

    # ---- checkpoint / resume ----------------------------------------------------------------------
    def snapshot(self):
        """Host copy of everything a later run needs, taken between two scheduler rounds (after a
        compact): the request table, token arena, block masks, row map, queue and active rows, plus
        the fixed parameters.  The box, per-row views and step buffers are rebuilt by the next pack."""
        h = self.host_table()
        return dict(h, rows=self.rows, L=self.L, V=self.V, dtype=self.dtype, rows_cap=self.rows_cap,
                    budget=self.budget, mask_id=self.mask_id, pad_id=self.pad_id, eos_id=self.eos_id)

    @classmethod
    def from_snapshot(cls, snap, device="cuda", logits=None):
        """A session that continues from snapshot(): run() then carries on where the other stopped
        (its opening admission admits nothing the last compact did not)."""
        return cls(snap["p"], snap["K"], snap["b"], snap["state"], snap["threshold"], snap["arena_off"],
                   snap["arena"], snap["blk_mask"], snap["row_req"], snap["rows"], snap["queue"], L=snap["L"],
                   V=snap["V"], dtype=snap["dtype"], rows_cap=snap["rows_cap"], budget=snap["budget"],
                   mask_id=snap["mask_id"], pad_id=snap["pad_id"], eos_id=snap["eos_id"], device=device,
                   logits=logits)

    # ---- host views for tests -----------------------------------------------------------------
    def host_table(self):
        """Host copies of the request table, row map and queue."""
        torch.cuda.synchronize()
        r = self.reqs
        qlen = int(self.queue.len.item())
        return dict(p=r.p.cpu().numpy(), K=r.K.cpu().numpy(), b=r.b.cpu().numpy(), state=r.state.cpu().numpy(),
                    threshold=r.threshold.cpu().numpy(), arena_off=r.arena_off.cpu().numpy(),
                    arena=r.arena.cpu().numpy(), blk_mask=r.blk_mask.cpu().numpy(),
                    row_req=self.row_req.cpu().numpy(), queue=self.queue.ids[:qlen].cpu().numpy())
