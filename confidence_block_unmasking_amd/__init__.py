"""MI355X-native dLLM denoise step: LowConfidence unmasking, mixed-state packing, FDFO compaction.

The compute lives in libdllm.so (HIP for gfx950, C ABI in include/dllm.h); this package is the
binding (api) and the host loop driver (driver).
"""
from ._lib import DllmError, EXPORTS, LIB_PATH, lib  # noqa: F401
from .api import (DevQueue, KernelEvents, ReqTable, dllm_compact, dllm_pack, dllm_step,  # noqa: F401
                  dllm_step_decide, dllm_step_decide_quota, dllm_step_decide_shards, dllm_step_features,
                  dllm_step_quota, dllm_step_score, dllm_step_score_shard, dllm_step_score_timed, dllm_step_timed,
                  dllm_step_workspace_bytes, new_triples, new_workspace, read_meta)
