"""Thin torch-facing binding of the C ABI: argument marshalling only.

Every function hands device pointers of caller-owned torch tensors to libdllm.so and enqueues work
on the current torch stream (or the stream given).  No part of the step, pack or compact
computation runs here.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import DllmError, Meta, Queue, Reqs  # noqa: F401  (re-exported)

_DT = {torch.bfloat16: _lib.DLLM_BF16, torch.float32: _lib.DLLM_FP32}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _launch(fn, args, where, events, stream):
    """Call fn(*args) and check its status; with `events` (two timing events), they are recorded on
    the launch stream right before and right after the call, after every argument is marshalled."""
    if events is not None:
        s = torch.cuda.current_stream() if stream is None else stream
        events[0].record(s)
        rc = fn(*args)
        events[1].record(s)
    else:
        rc = fn(*args)
    _lib.check(rc, where)


def _need(t, dtype, name, numel=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")


def dllm_step_workspace_bytes(rows: int, L: int, V: int, dtype=torch.bfloat16) -> int:
    return int(_lib.lib().dllm_step_workspace_bytes(rows, L, V, _DT[dtype]))


def new_workspace(rows: int, L: int, V: int, dtype=torch.bfloat16, device="cuda"):
    """A step workspace for this shape (the step needs no particular contents; zero-filled here)."""
    n = dllm_step_workspace_bytes(rows, L, V, dtype)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def _logits_shape(logits, rows, L, V, pos_stride, row_stride):
    """Shape and strides (in elements) of the logits; the kernels read element (r, j, v) at
    r*row_stride + j*pos_stride + v, so the tensor's storage must reach that far."""
    if logits.dtype not in _DT:
        raise ValueError(f"logits dtype {logits.dtype} not supported")
    # the kernels read a slot's V elements as one contiguous run
    if logits.dim() >= 1 and logits.shape[-1] > 1 and logits.stride(-1) != 1:
        raise ValueError(f"logits must have unit stride along the vocabulary, got stride {logits.stride(-1)}")
    if not logits.is_cuda:
        raise ValueError("logits must be a device tensor")
    if rows is None:
        rows, L, V = logits.shape
    if pos_stride is None:
        pos_stride = logits.stride(1) if logits.dim() == 3 else V
    if row_stride is None:
        row_stride = logits.stride(0) if logits.dim() == 3 else L * pos_stride
    if rows > 0 and L > 0 and V > 0:
        reach = (rows - 1) * row_stride + (L - 1) * pos_stride + V
        avail = logits.untyped_storage().nbytes() // logits.element_size() - logits.storage_offset()
        if reach > avail:
            raise ValueError(f"logits storage holds {avail} elements past its offset; rows={rows}, L={L}, V={V} "
                             f"with strides ({row_stride}, {pos_stride}) reach {reach}")
    return rows, L, V, pos_stride, row_stride


def _decide_args(rows, L, input_ids, mask_in, mask_out, threshold, done, accept_len, workspace, status, p, b, conf,
                 argmax, need_tau=True):
    W = input_ids.shape[-1]
    _need(input_ids, torch.int32, "input_ids", rows * W)
    _need(mask_in, torch.uint8, "mask_in", rows * L)
    _need(mask_out, torch.uint8, "mask_out", rows * L)
    if need_tau:
        _need(threshold, torch.float32, "threshold", rows)
    _need(done, torch.uint8, "done", rows)
    _need(accept_len, torch.int32, "accept_len", rows)
    _need(workspace, torch.uint8, "workspace")
    _need(status, torch.int32, "status", 1)
    for t, dt, nm, n in ((p, torch.int32, "p", rows), (b, torch.int32, "b", rows),
                         (conf, torch.float32, "conf", rows * L), (argmax, torch.int32, "argmax", rows * L)):
        if t is not None:
            _need(t, dt, nm, n)
    return W


def dllm_step(logits, input_ids, mask_in, mask_out, threshold, done, accept_len, workspace, status,
              p=None, b=None, conf=None, argmax=None, rows=None, L=None, V=None, pos_stride=None,
              row_stride=None, stream=None, events=None):
    """One LowConfidence denoise step (see include/dllm.h).

    logits: [rows, L, V] bf16/fp32 device tensor, or any tensor whose storage holds element
    (r, j, v) at r*row_stride + j*pos_stride + v when the strides are given.  events: optional
    pair of timing events recorded right around the library call.
    """
    rows, L, V, pos_stride, row_stride = _logits_shape(logits, rows, L, V, pos_stride, row_stride)
    W = _decide_args(rows, L, input_ids, mask_in, mask_out, threshold, done, accept_len, workspace, status, p, b,
                     conf, argmax)
    args = (_stream(stream), _ptr(logits), _DT[logits.dtype], pos_stride, row_stride, rows, L, V, _ptr(input_ids), W,
            _ptr(mask_in), _ptr(mask_out), _ptr(threshold), _ptr(p), _ptr(b), _ptr(conf), _ptr(argmax), _ptr(done),
            _ptr(accept_len), _ptr(workspace), workspace.numel(), _ptr(status))
    _launch(_lib.lib().dllm_step, args, "dllm_step", events, stream)


def dllm_step_noalloc(logits, input_ids, mask_in, mask_out, threshold, done, accept_len, status, p=None, b=None,
                      conf=None, argmax=None, rows=None, L=None, V=None, pos_stride=None, row_stride=None, stream=None):
    """dllm_step without a workspace: the library's fixed per-device scratch holds the partials
    (for callers that cannot allocate; calls on one GPU must not overlap).  See include/dllm.h."""
    rows, L, V, pos_stride, row_stride = _logits_shape(logits, rows, L, V, pos_stride, row_stride)
    W = input_ids.shape[-1]
    _need(input_ids, torch.int32, "input_ids", rows * W)
    _need(mask_in, torch.uint8, "mask_in", rows * L)
    _need(mask_out, torch.uint8, "mask_out", rows * L)
    _need(threshold, torch.float32, "threshold", rows)
    _need(done, torch.uint8, "done", rows)
    _need(accept_len, torch.int32, "accept_len", rows)
    _need(status, torch.int32, "status", 1)
    for t, dt, nm, n in ((p, torch.int32, "p", rows), (b, torch.int32, "b", rows),
                         (conf, torch.float32, "conf", rows * L), (argmax, torch.int32, "argmax", rows * L)):
        if t is not None:
            _need(t, dt, nm, n)
    rc = _lib.lib().dllm_step_noalloc(_stream(stream), _ptr(logits), _DT[logits.dtype], pos_stride, row_stride, rows,
                                      L, V, _ptr(input_ids), W, _ptr(mask_in), _ptr(mask_out), _ptr(threshold),
                                      _ptr(p), _ptr(b), _ptr(conf), _ptr(argmax), _ptr(done), _ptr(accept_len),
                                      _ptr(status))
    _lib.check(rc, "dllm_step_noalloc")


def dllm_step_timed(logits, input_ids, mask_in, mask_out, threshold, done, accept_len, workspace, status, kernel_events,
                    p=None, b=None, conf=None, argmax=None, rows=None, L=None, V=None, pos_stride=None,
                    row_stride=None, stream=None):
    """dllm_step with `kernel_events` (a KernelEvents) bound to the scoring kernel's start and the
    deciding kernel's end."""
    rows, L, V, pos_stride, row_stride = _logits_shape(logits, rows, L, V, pos_stride, row_stride)
    W = _decide_args(rows, L, input_ids, mask_in, mask_out, threshold, done, accept_len, workspace, status, p, b,
                     conf, argmax)
    args = (_stream(stream), _ptr(logits), _DT[logits.dtype], pos_stride, row_stride, rows, L, V, _ptr(input_ids), W,
            _ptr(mask_in), _ptr(mask_out), _ptr(threshold), _ptr(p), _ptr(b), _ptr(conf), _ptr(argmax), _ptr(done),
            _ptr(accept_len), _ptr(workspace), workspace.numel(), _ptr(status), kernel_events.start,
            kernel_events.stop)
    _launch(_lib.lib().dllm_step_timed, args, "dllm_step_timed", None, stream)


def dllm_step_score(logits, mask_in, workspace, status, rows=None, L=None, V=None, pos_stride=None,
                    row_stride=None, stream=None):
    """The scoring half of dllm_step: per-chunk partials of every masked slot into `workspace`."""
    rows, L, V, pos_stride, row_stride = _logits_shape(logits, rows, L, V, pos_stride, row_stride)
    _need(mask_in, torch.uint8, "mask_in", rows * L)
    _need(workspace, torch.uint8, "workspace")
    _need(status, torch.int32, "status", 1)
    rc = _lib.lib().dllm_step_score(_stream(stream), _ptr(logits), _DT[logits.dtype], pos_stride, row_stride, rows,
                                    L, V, _ptr(mask_in), _ptr(workspace), workspace.numel(), _ptr(status))
    _lib.check(rc, "dllm_step_score")


class KernelEvents:
    """Two HIP events with timing enabled, for dllm_step_score_timed.  They are created through the
    HIP runtime that libdllm.so and torch share; elapsed_ms() waits for the second one."""

    def __init__(self):
        hip = _lib.lib()
        self._hip = hip
        self.start, self.stop = ctypes.c_void_p(), ctypes.c_void_p()
        for e in (self.start, self.stop):
            if hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")

    def elapsed_ms(self) -> float:
        if self._hip.hipEventSynchronize(self.stop) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.start, self.stop) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        for e in (getattr(self, "start", None), getattr(self, "stop", None)):
            if e is not None and e.value:
                self._hip.hipEventDestroy(e)


def dllm_step_score_timed(logits, mask_in, workspace, status, events, rows=None, L=None, V=None, pos_stride=None,
                          row_stride=None, stream=None):
    """dllm_step_score with the scoring kernel's own start and end recorded into `events`
    (a KernelEvents)."""
    rows, L, V, pos_stride, row_stride = _logits_shape(logits, rows, L, V, pos_stride, row_stride)
    _need(mask_in, torch.uint8, "mask_in", rows * L)
    _need(workspace, torch.uint8, "workspace")
    _need(status, torch.int32, "status", 1)
    rc = _lib.lib().dllm_step_score_timed(_stream(stream), _ptr(logits), _DT[logits.dtype], pos_stride, row_stride,
                                          rows, L, V, _ptr(mask_in), _ptr(workspace), workspace.numel(),
                                          _ptr(status), events.start, events.stop)
    _lib.check(rc, "dllm_step_score_timed")


def dllm_step_decide(dtype, rows, L, V, input_ids, mask_in, mask_out, threshold, done, accept_len, workspace, status,
                     p=None, b=None, conf=None, argmax=None, unmasked=None, fallback=None, stream=None, events=None):
    """The deciding half of dllm_step, on the partials dllm_step_score left in `workspace`
    (same dtype, rows, L, V and mask_in).  unmasked (int32 [rows]) and fallback (uint8 [rows]),
    when given, receive each row's count of slots unmasked and whether the rule's single-slot
    fallback applied.  events: optional pair of timing events recorded right around the call."""
    if dtype not in _DT:
        raise ValueError(f"dtype {dtype} not supported")
    W = _decide_args(rows, L, input_ids, mask_in, mask_out, threshold, done, accept_len, workspace, status, p, b,
                     conf, argmax)
    if unmasked is not None:
        _need(unmasked, torch.int32, "unmasked", rows)
    if fallback is not None:
        _need(fallback, torch.uint8, "fallback", rows)
    args = (_stream(stream), _DT[dtype], rows, L, V, _ptr(input_ids), W, _ptr(mask_in), _ptr(mask_out),
            _ptr(threshold), _ptr(p), _ptr(b), _ptr(conf), _ptr(argmax), _ptr(done), _ptr(accept_len),
            _ptr(workspace), workspace.numel(), _ptr(status), _ptr(unmasked), _ptr(fallback))
    _launch(_lib.lib().dllm_step_decide, args, "dllm_step_decide", events, stream)


def dllm_step_quota(logits, input_ids, mask_in, mask_out, steps_per_block, done, accept_len, workspace, status,
                    p=None, b=None, conf=None, argmax=None, rows=None, L=None, V=None, pos_stride=None,
                    row_stride=None, stream=None):
    """One denoise step with the fixed per-step quota (steps_per_block diffusion steps per block)."""
    rows, L, V, pos_stride, row_stride = _logits_shape(logits, rows, L, V, pos_stride, row_stride)
    W = _decide_args(rows, L, input_ids, mask_in, mask_out, None, done, accept_len, workspace, status, p, b, conf,
                     argmax, need_tau=False)
    rc = _lib.lib().dllm_step_quota(_stream(stream), _ptr(logits), _DT[logits.dtype], pos_stride, row_stride, rows,
                                    L, V, _ptr(input_ids), W, _ptr(mask_in), _ptr(mask_out), int(steps_per_block),
                                    _ptr(p), _ptr(b), _ptr(conf), _ptr(argmax), _ptr(done), _ptr(accept_len),
                                    _ptr(workspace), workspace.numel(), _ptr(status))
    _lib.check(rc, "dllm_step_quota")


def dllm_step_decide_quota(dtype, rows, L, V, input_ids, mask_in, mask_out, steps_per_block, done, accept_len,
                           workspace, status, p=None, b=None, conf=None, argmax=None, stream=None):
    """The deciding half of dllm_step_quota, on the partials dllm_step_score left in `workspace`."""
    if dtype not in _DT:
        raise ValueError(f"dtype {dtype} not supported")
    W = _decide_args(rows, L, input_ids, mask_in, mask_out, None, done, accept_len, workspace, status, p, b, conf,
                     argmax, need_tau=False)
    rc = _lib.lib().dllm_step_decide_quota(_stream(stream), _DT[dtype], rows, L, V, _ptr(input_ids), W,
                                           _ptr(mask_in), _ptr(mask_out), int(steps_per_block), _ptr(p), _ptr(b),
                                           _ptr(conf), _ptr(argmax), _ptr(done), _ptr(accept_len), _ptr(workspace),
                                           workspace.numel(), _ptr(status))
    _lib.check(rc, "dllm_step_decide_quota")


def new_triples(rows: int, L: int, n_shards: int, device="cuda"):
    """Buffer for the per-shard results of dllm_step_score_shard ([rows, L, n_shards] records of 16 B)."""
    n = _lib.lib().dllm_shard_triples_bytes(rows, L, n_shards)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device)


def dllm_step_score_shard(logits, mask_in, workspace, triples, shard, n_shards, vocab_offset, status, rows=None,
                          L=None, V_shard=None, pos_stride=None, row_stride=None, stream=None):
    """Score one vocabulary shard (columns vocab_offset .. + V_shard - 1) of every masked slot."""
    rows, L, V_shard, pos_stride, row_stride = _logits_shape(logits, rows, L, V_shard, pos_stride, row_stride)
    _need(mask_in, torch.uint8, "mask_in", rows * L)
    _need(workspace, torch.uint8, "workspace")
    _need(triples, torch.uint8, "triples", _lib.lib().dllm_shard_triples_bytes(rows, L, n_shards))
    _need(status, torch.int32, "status", 1)
    rc = _lib.lib().dllm_step_score_shard(_stream(stream), _ptr(logits), _DT[logits.dtype], pos_stride, row_stride,
                                          rows, L, V_shard, int(vocab_offset), int(shard), int(n_shards),
                                          _ptr(mask_in), _ptr(workspace), workspace.numel(), _ptr(triples),
                                          _ptr(status))
    _lib.check(rc, "dllm_step_score_shard")


def dllm_step_decide_shards(n_shards, triples, rows, L, V, input_ids, mask_in, mask_out, threshold, done, accept_len,
                            status, p=None, b=None, conf=None, argmax=None, stream=None):
    """Combine the shards' results per masked slot and apply the LowConfidence rule."""
    W = _decide_args(rows, L, input_ids, mask_in, mask_out, threshold, done, accept_len, triples, status, p, b, conf,
                     argmax)
    _need(triples, torch.uint8, "triples", _lib.lib().dllm_shard_triples_bytes(rows, L, n_shards))
    rc = _lib.lib().dllm_step_decide_shards(_stream(stream), int(n_shards), _ptr(triples), rows, L, V,
                                            _ptr(input_ids), W, _ptr(mask_in), _ptr(mask_out), _ptr(threshold),
                                            _ptr(p), _ptr(b), _ptr(conf), _ptr(argmax), _ptr(done), _ptr(accept_len),
                                            _ptr(status))
    _lib.check(rc, "dllm_step_decide_shards")


N_FEATURES = 9


def dllm_step_features(rows, L, row_req, reqs: "ReqTable", conf, mask_out, features, status, stream=None):
    """Step-predictor features per row after a step: float32 [rows, 9] (see include/dllm.h)."""
    _need(row_req, torch.int32, "row_req", rows)
    _need(conf, torch.float32, "conf", rows * L)
    _need(mask_out, torch.uint8, "mask_out", rows * L)
    _need(features, torch.float32, "features", rows * N_FEATURES)
    _need(status, torch.int32, "status", 1)
    st = reqs.struct()
    rc = _lib.lib().dllm_step_features(_stream(stream), rows, L, _ptr(row_req), ctypes.byref(st), _ptr(conf),
                                       _ptr(mask_out), _ptr(features), _ptr(status))
    _lib.check(rc, "dllm_step_features")


class ReqTable:
    """Device-resident request table (the fields of dllm_reqs), built from host numpy arrays."""

    def __init__(self, p, K, b, state, threshold, arena_off, arena, blk_mask, device="cuda"):
        def dev(a, dt):
            return torch.as_tensor(a).to(dtype=dt).contiguous().to(device)
        self.p = dev(p, torch.int32)
        self.K = dev(K, torch.int32)
        self.b = dev(b, torch.int32)
        self.state = dev(state, torch.int32)
        self.threshold = dev(threshold, torch.float32)
        self.arena_off = dev(arena_off, torch.int64)
        self.arena = dev(arena, torch.int32)
        self.blk_mask = dev(blk_mask, torch.uint8)
        self.L = int(self.blk_mask.shape[1])
        self.n_req = int(self.p.shape[0])

    def struct(self) -> Reqs:
        return Reqs(self.n_req, self.p.data_ptr(), self.K.data_ptr(), self.b.data_ptr(), self.state.data_ptr(),
                    self.threshold.data_ptr(), self.arena_off.data_ptr(), self.arena.data_ptr(),
                    self.blk_mask.data_ptr())


class DevQueue:
    """Device-resident pending queue (dllm_queue): ids [cap] and a device length."""

    def __init__(self, ids, device="cuda", cap=None):
        ids = torch.as_tensor(ids).to(torch.int32)
        cap = int(ids.numel()) if cap is None else int(cap)
        self.ids = torch.full((max(cap, 1),), -1, dtype=torch.int32, device=device)
        self.ids[:ids.numel()] = ids.to(device)
        self.len = torch.tensor([ids.numel()], dtype=torch.int32, device=device)
        self.cap = cap

    def struct(self) -> Queue:
        return Queue(self.ids.data_ptr(), self.len.data_ptr(), self.cap)


def dllm_pack(rows, L, W, pad_id, row_req, reqs: ReqTable, box_ids, mask, threshold, p, b, status,
              box_valid=None, box_pos=None, stream=None, events=None):
    """Gather the left-padded box for rows [0, rows) (see include/dllm.h).  events: optional pair
    of timing events recorded right around the library call."""
    if rows > 0:
        _need(row_req, torch.int32, "row_req", rows)
        _need(box_ids, torch.int32, "box_ids", rows * W)
        _need(mask, torch.uint8, "mask", rows * L)
        _need(threshold, torch.float32, "threshold", rows)
        _need(p, torch.int32, "p", rows)
        _need(b, torch.int32, "b", rows)
        _need(status, torch.int32, "status", 1)
        if box_valid is not None:
            _need(box_valid, torch.uint8, "box_valid", rows * W)
        if box_pos is not None:
            _need(box_pos, torch.int32, "box_pos", rows * W)
    st = reqs.struct()
    args = (_stream(stream), rows, L, W, pad_id, _ptr(row_req), ctypes.byref(st), _ptr(box_ids), _ptr(box_valid),
            _ptr(box_pos), _ptr(mask), _ptr(threshold), _ptr(p), _ptr(b), _ptr(status))
    _launch(_lib.lib().dllm_pack, args, "dllm_pack", events, stream)


def dllm_compact(rows, L, W, mask_id, eos_id, row_req, rows_cap, reqs: ReqTable, queue: DevQueue, budget, meta,
                 status, box_ids=None, mask=None, done=None, stream=None, events=None):
    """Commit finished blocks, evict, refill under the token budget (see include/dllm.h).
    meta: device uint8 tensor of 32 bytes (a dllm_meta).  events: optional pair of timing events
    recorded right around the library call."""
    _need(row_req, torch.int32, "row_req", rows_cap)
    _need(meta, torch.uint8, "meta", 32)
    _need(status, torch.int32, "status", 1)
    if box_ids is not None:
        _need(box_ids, torch.int32, "box_ids", rows * W)
        _need(mask, torch.uint8, "mask", rows * L)
        _need(done, torch.uint8, "done", rows)
    st = reqs.struct()
    q = queue.struct()
    args = (_stream(stream), rows, L, W, mask_id, eos_id, _ptr(box_ids), _ptr(mask), _ptr(done), _ptr(row_req),
            rows_cap, ctypes.byref(st), ctypes.byref(q), int(budget), _ptr(meta), _ptr(status))
    _launch(_lib.lib().dllm_compact, args, "dllm_compact", events, stream)


def read_meta(meta_tensor) -> dict:
    """Copy a device dllm_meta to the host (synchronises with the tensor's stream)."""
    raw = meta_tensor.cpu().numpy().tobytes()
    m = Meta.from_buffer_copy(raw)
    return dict(rows=m.rows, W=m.W, n_evicted=m.n_evicted, n_admitted=m.n_admitted, n_queued=m.n_queued,
                cost=m.cost)
