"""The C ABI from C (no GPU): include/dllm.h compiles as strict C99 and as C++17; a C program that
takes the address of every declared entry point links against libdllm.so; its structs have the
layout the ctypes binding mirrors, its limits are the binding's, and the host-only calls behave as
the header states (workspace size, synchronous argument errors with text)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

from confidence_block_unmasking_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
PKG = os.path.dirname(_lib.LIB_PATH)

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc and g++")


def _declared():
    src = open(os.path.join(INC, "dllm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dllm_\w+)\s*\(", src)))


def _program():
    fns = ",\n        ".join(f"(anyfn){n}" for n in _declared())
    return r"""
#include <stddef.h>
#include <stdio.h>
#include "dllm.h"

typedef void (*anyfn)(void);

int main(void) {
    anyfn fns[] = {
        %s
    };
    size_t k, n_null = 0;
    for (k = 0; k < sizeof fns / sizeof fns[0]; ++k) n_null += fns[k] == NULL;
    printf("entry_points %%zu null %%zu\n", sizeof fns / sizeof fns[0], n_null);
    printf("reqs %%zu %%zu %%zu %%zu %%zu %%zu %%zu %%zu %%zu %%zu\n", sizeof(dllm_reqs),
           offsetof(dllm_reqs, n_req), offsetof(dllm_reqs, p), offsetof(dllm_reqs, K), offsetof(dllm_reqs, b),
           offsetof(dllm_reqs, state), offsetof(dllm_reqs, threshold), offsetof(dllm_reqs, arena_off),
           offsetof(dllm_reqs, arena), offsetof(dllm_reqs, blk_mask));
    printf("queue %%zu %%zu %%zu %%zu\n", sizeof(dllm_queue), offsetof(dllm_queue, ids),
           offsetof(dllm_queue, len), offsetof(dllm_queue, cap));
    printf("meta %%zu %%zu %%zu %%zu %%zu %%zu %%zu %%zu\n", sizeof(dllm_meta), offsetof(dllm_meta, rows),
           offsetof(dllm_meta, W), offsetof(dllm_meta, n_evicted), offsetof(dllm_meta, n_admitted),
           offsetof(dllm_meta, n_queued), offsetof(dllm_meta, reserved), offsetof(dllm_meta, cost));
    printf("limits %%d %%d %%d %%d %%d %%zu\n", DLLM_MAX_L, DLLM_MAX_ROWS, DLLM_MAX_POSITIONS, DLLM_MAX_QUEUE,
           DLLM_MAX_SHARDS, DLLM_NOALLOC_SCRATCH_BYTES);
    printf("codes %%d %%d %%d %%d %%d %%d %%d %%d\n", DLLM_OK, DLLM_ERR_ARG, DLLM_ERR_SHAPE, DLLM_ERR_DTYPE,
           DLLM_ERR_CAPACITY, DLLM_ERR_HIP, DLLM_FP32, DLLM_BF16);
    printf("workspace %%zu %%zu\n", dllm_step_workspace_bytes(64, 32, 152064, DLLM_BF16),
           dllm_step_workspace_bytes(64, 32, 152064, 7));
    {
        /* a null logits pointer is rejected before anything reaches a device */
        dllm_status rc = dllm_step(NULL, NULL, DLLM_BF16, 152064, 32 * 152064, 64, 32, 152064, NULL, 600, NULL,
                                   NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL);
        printf("step_null %%d %%s\n", (int)rc, dllm_last_error());
    }
    {
        int32_t dummy = 0;
        dllm_status rc = dllm_pack(NULL, 4, 0, 64, 0, &dummy, NULL, &dummy, NULL, NULL, NULL, NULL, &dummy, &dummy,
                                   &dummy);
        printf("pack_badL %%d %%s\n", (int)rc, dllm_last_error());
    }
    return 0;
}
""" % fns


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


@pytest.fixture(scope="module")
def c_program(tmp_path_factory):
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libdllm.so is not built")
    d = tmp_path_factory.mktemp("capi")
    src = d / "use_dllm.c"
    src.write_text(_program())
    exe = d / "use_dllm"
    _run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-Wno-cast-function-type", "-I", INC,
          str(src), "-L", PKG, "-ldllm", f"-Wl,-rpath,{PKG}", "-Wl,--allow-shlib-undefined", "-o", str(exe)])
    env = dict(os.environ)
    # the HIP runtime the library needs is where torch found it
    import torch  # noqa: F401
    env["LD_LIBRARY_PATH"] = os.pathsep.join(
        [p for p in [os.path.join(os.path.dirname(torch.__file__), "lib"), "/opt/rocm/lib",
                     env.get("LD_LIBRARY_PATH", "")] if p])
    out = _run([str(exe)], env=env)
    return {ln.split()[0]: ln.split()[1:] for ln in out.strip().splitlines()}


def test_header_is_strict_c99_and_cxx17(tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "dllm.h"\nint dllm_header_only;\n')
    _run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-I", INC, str(src)])
    cxx = tmp_path / "h.cc"
    cxx.write_text('#include "dllm.h"\nstatic_assert(sizeof(dllm_meta) == 32, "meta");\nint dllm_header_only;\n')
    _run(["g++", "-std=c++17", "-pedantic", "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-I", INC, str(cxx)])


def test_every_entry_point_links_from_c(c_program):
    n, n_null = c_program["entry_points"][0], c_program["entry_points"][2]
    assert int(n) == len(_lib.EXPORTS) and int(n_null) == 0


def test_struct_layouts_match_the_binding(c_program):
    for cname, cls in (("reqs", _lib.Reqs), ("queue", _lib.Queue), ("meta", _lib.Meta)):
        got = [int(v) for v in c_program[cname]]
        assert got[0] == ctypes.sizeof(cls), cname
        assert got[1:] == [getattr(cls, f).offset for f, _ in cls._fields_], cname


def test_limits_and_codes_match_the_binding(c_program):
    assert [int(v) for v in c_program["limits"]] == [_lib.MAX_L, _lib.MAX_ROWS, _lib.MAX_POSITIONS,
                                                     _lib.MAX_QUEUE, 1024, _lib.NOALLOC_SCRATCH_BYTES]
    assert [int(v) for v in c_program["codes"]] == [_lib.DLLM_OK, _lib.DLLM_ERR_ARG, _lib.DLLM_ERR_SHAPE,
                                                    _lib.DLLM_ERR_DTYPE, _lib.DLLM_ERR_CAPACITY, _lib.DLLM_ERR_HIP,
                                                    _lib.DLLM_FP32, _lib.DLLM_BF16]


def test_host_only_calls_from_c(c_program):
    ws, bad = (int(v) for v in c_program["workspace"])
    assert ws == _lib.lib().dllm_step_workspace_bytes(64, 32, 152064, _lib.DLLM_BF16) and ws >= 64 * 32 * 38 * 16
    assert bad == 0
    rc, *text = c_program["step_null"]
    assert int(rc) == _lib.DLLM_ERR_ARG and "dllm_step" in " ".join(text)
    rc, *text = c_program["pack_badL"]
    assert int(rc) == _lib.DLLM_ERR_SHAPE and "L=0" in " ".join(text)
