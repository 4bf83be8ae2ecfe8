"""Bindings for the synthetic logits generator (CPU: synth.c, GPU: synth_gpu.hip).

The generator's definition is written out at the top of synth.c and synth_gpu.hip.  It only
produces inputs; the unmasking method itself is not computed here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
CPU_LIB = os.path.join(HERE, "libsynth_cpu.so")
GPU_LIB = os.path.join(HERE, "libsynth_gpu.so")
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose=False):
    """Compile both generator libraries in place (always recompiles)."""
    cmds = [
        ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-o", CPU_LIB, os.path.join(HERE, "synth.c")],
        ["hipcc", *HIP_FLAGS, "-o", GPU_LIB, os.path.join(HERE, "synth_gpu.hip")],
    ]
    for c in cmds:
        if verbose:
            print(" ".join(c), flush=True)
        subprocess.run(c, check=True)


_cpu = None
_gpu = None


def _cpu_lib():
    global _cpu
    if _cpu is None:
        if not os.path.exists(CPU_LIB):
            build()
        lib = ctypes.CDLL(CPU_LIB)
        lib.synth_logits_cpu.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int]
        lib.synth_logits_cpu.restype = None
        lib.synth_row_cpu.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_uint64,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int32, ctypes.c_int32]
        lib.synth_row_cpu.restype = None
        lib.synth_planted_cpu.argtypes = [ctypes.c_int32, ctypes.c_uint64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int64]
        lib.synth_planted_cpu.restype = ctypes.c_int64
        _cpu = lib
    return _cpu


def _gpu_lib():
    global _gpu
    if _gpu is None:
        if not os.path.exists(GPU_LIB):
            raise RuntimeError(f"{GPU_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(GPU_LIB)
        lib.synth_logits_gpu.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int]
        lib.synth_logits_gpu.restype = ctypes.c_int
        _gpu = lib
    return _gpu


def _dt(dtype):
    return {"fp32": 0, "bf16": 1}[dtype]


def logits_cpu(rows, L, V, dtype, row_req, blk, mask, seed, sigma, umax, fill_nan=True, out=None):
    """Host logits [rows, L, V]: float32 for fp32, uint16 bit patterns for bf16."""
    row_req = np.ascontiguousarray(row_req[:rows], np.int32)
    blk = np.ascontiguousarray(blk[:rows], np.int32)
    mask = np.ascontiguousarray(mask[:rows], np.uint8)
    if out is None:
        out = np.empty((rows, L, V), np.float32 if dtype == "fp32" else np.uint16)
    assert out.flags.c_contiguous and out.shape[1:] == (L, V)
    _cpu_lib().synth_logits_cpu(out.ctypes.data, _dt(dtype), V, L * V, rows, L, V, row_req.ctypes.data,
                                blk.ctypes.data, mask.ctypes.data, seed, sigma, umax, int(fill_nan))
    return out


def row_cpu(V, dtype, seed, req, block, j, m_rem, sigma, umax):
    """One vocabulary row for (req, block, slot j) when m_rem slots of the block are masked."""
    out = np.empty(V, np.float32 if dtype == "fp32" else np.uint16)
    _cpu_lib().synth_row_cpu(out.ctypes.data, _dt(dtype), V, seed, req, block, j, m_rem, sigma, umax)
    return out


def planted_cpu(V, seed, req, block, j):
    return int(_cpu_lib().synth_planted_cpu(V, seed, req, block, j))


def logits_gpu(out, dtype, rows, L, V, row_req, blk, mask, seed, sigma, umax, fill_nan=False,
               pos_stride=None, row_stride=None, stream=None):
    """Fill a device tensor `out` (torch, element layout r*row_stride + j*pos_stride + v)."""
    import torch
    pos_stride = V if pos_stride is None else pos_stride
    row_stride = L * pos_stride if row_stride is None else row_stride
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream
    rc = _gpu_lib().synth_logits_gpu(ctypes.c_void_p(s), ctypes.c_void_p(out.data_ptr()), _dt(dtype),
                                     pos_stride, row_stride, rows, L, V, ctypes.c_void_p(row_req.data_ptr()),
                                     ctypes.c_void_p(blk.data_ptr()), ctypes.c_void_p(mask.data_ptr()),
                                     seed, sigma, umax, int(fill_nan))
    if rc != 0:
        raise RuntimeError(f"synth_logits_gpu failed with code {rc}")

