"""ctypes loader for libdllm.so (the C ABI declared in include/dllm.h).

Loads the in-tree library built by confidence_block_unmasking_amd/build.py and fails loudly when
it is missing: there is no fallback implementation of any entry point.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdllm.so")

DLLM_OK, DLLM_ERR_ARG, DLLM_ERR_SHAPE, DLLM_ERR_DTYPE, DLLM_ERR_CAPACITY, DLLM_ERR_HIP = range(6)
STATUS_NAMES = {0: "DLLM_OK", 1: "DLLM_ERR_ARG", 2: "DLLM_ERR_SHAPE", 3: "DLLM_ERR_DTYPE",
                4: "DLLM_ERR_CAPACITY", 5: "DLLM_ERR_HIP"}
DLLM_FP32, DLLM_BF16 = 0, 1
MAX_L, MAX_ROWS, MAX_POSITIONS, MAX_QUEUE = 1024, 4096, 262144, 8192
NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTS = ("dllm_step", "dllm_step_noalloc", "dllm_step_timed", "dllm_step_score", "dllm_step_score_timed", "dllm_step_decide", "dllm_step_quota", "dllm_step_decide_quota",
           "dllm_step_features", "dllm_step_score_shard", "dllm_step_decide_shards", "dllm_shard_triples_bytes",
           "dllm_step_workspace_bytes", "dllm_pack", "dllm_compact", "dllm_last_error")


class DllmError(RuntimeError):
    def __init__(self, code, where, text=""):
        self.code = code
        super().__init__(f"{where}: {STATUS_NAMES.get(code, code)} {text}".strip())


class Reqs(ctypes.Structure):
    _fields_ = [("n_req", ctypes.c_int32), ("p", ctypes.c_void_p), ("K", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("state", ctypes.c_void_p), ("threshold", ctypes.c_void_p), ("arena_off", ctypes.c_void_p),
                ("arena", ctypes.c_void_p), ("blk_mask", ctypes.c_void_p)]


class Queue(ctypes.Structure):
    _fields_ = [("ids", ctypes.c_void_p), ("len", ctypes.c_void_p), ("cap", ctypes.c_int32)]


class Meta(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("W", ctypes.c_int32), ("n_evicted", ctypes.c_int32),
                ("n_admitted", ctypes.c_int32), ("n_queued", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("cost", ctypes.c_int64)]


assert ctypes.sizeof(Meta) == 32

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: build it with confidence_block_unmasking_amd/build.py "
                               "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.dllm_step.argtypes = [vp, vp, i32, i64, i64, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp,
                                vp, vp, vp, sz, vp]
        L.dllm_step.restype = i32
        L.dllm_step_noalloc.argtypes = [vp, vp, i32, i64, i64, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp]
        L.dllm_step_noalloc.restype = i32
        L.dllm_step_timed.argtypes = [vp, vp, i32, i64, i64, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp, vp, sz, vp, vp, vp]
        L.dllm_step_timed.restype = i32
        L.dllm_step_score.argtypes = [vp, vp, i32, i64, i64, i32, i32, i32, vp, vp, sz, vp]
        L.dllm_step_score.restype = i32
        L.dllm_step_score_timed.argtypes = [vp, vp, i32, i64, i64, i32, i32, i32, vp, vp, sz, vp, vp, vp]
        L.dllm_step_score_timed.restype = i32
        L.dllm_step_decide.argtypes = [vp, i32, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       vp, sz, vp, vp, vp]
        L.dllm_step_decide.restype = i32
        L.dllm_step_quota.argtypes = [vp, vp, i32, i64, i64, i32, i32, i32, vp, i32, vp, vp, i32, vp, vp, vp,
                                      vp, vp, vp, vp, sz, vp]
        L.dllm_step_quota.restype = i32
        L.dllm_step_decide_quota.argtypes = [vp, i32, i32, i32, i32, vp, i32, vp, vp, i32, vp, vp, vp, vp,
                                             vp, vp, vp, sz, vp]
        L.dllm_step_decide_quota.restype = i32
        L.dllm_step_features.argtypes = [vp, i32, i32, vp, ctypes.POINTER(Reqs), vp, vp, vp, vp]
        L.dllm_step_features.restype = i32
        L.dllm_shard_triples_bytes.argtypes = [i32, i32, i32]
        L.dllm_shard_triples_bytes.restype = sz
        L.dllm_step_score_shard.argtypes = [vp, vp, i32, i64, i64, i32, i32, i32, i32, i32, i32, vp, vp, sz,
                                            vp, vp]
        L.dllm_step_score_shard.restype = i32
        L.dllm_step_decide_shards.argtypes = [vp, i32, vp, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                              vp]
        L.dllm_step_decide_shards.restype = i32
        L.dllm_step_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.dllm_step_workspace_bytes.restype = sz
        L.dllm_pack.argtypes = [vp, i32, i32, i32, i32, vp, ctypes.POINTER(Reqs), vp, vp, vp, vp, vp, vp, vp, vp]
        L.dllm_pack.restype = i32
        L.dllm_compact.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, i32, ctypes.POINTER(Reqs),
                                   ctypes.POINTER(Queue), i64, vp, vp]
        L.dllm_compact.restype = i32
        # the HIP runtime's event calls, reached through this library's own dependency (the same
        # runtime torch uses), for the kernel-bound timing of dllm_step_score_timed
        L.hipEventCreate.argtypes = [ctypes.POINTER(vp)]
        L.hipEventSynchronize.argtypes = [vp]
        L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        L.hipEventDestroy.argtypes = [vp]
        for f in (L.hipEventCreate, L.hipEventSynchronize, L.hipEventElapsedTime, L.hipEventDestroy):
            f.restype = ctypes.c_int
        L.dllm_last_error.argtypes = []
        L.dllm_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().dllm_last_error().decode(errors="replace")


def check(code: int, where: str):
    if code != DLLM_OK:
        raise DllmError(code, where, last_error())
