"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* libdllm.so's host side (argument checks, error text, shape and workspace arithmetic): a copy
  built with both sanitizers on the host pass only (device code is compiled as usual, and never
  runs here) is loaded in a child process with clang's sanitizer runtime preloaded, and runs the
  C ABI tests of test_abi.py, none of which reaches a device.
* The seeded CPU generator (workload/synth.c), built with gcc's sanitizers, runs the generator
  tests of test_workload.py.

Each child writes any sanitizer report to a log file and stops at the first one; the test fails
on a non-zero exit or on any report.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "confidence_block_unmasking_amd", "csrc")


def _clang_asan_runtime():
    try:
        res = subprocess.run(["hipcc", "--print-resource-dir"], capture_output=True, text=True, timeout=60)
    except (OSError, subprocess.TimeoutExpired):
        return None
    hits = glob.glob(os.path.join(res.stdout.strip(), "lib", "*", "libclang_rt.asan-x86_64.so"))
    return hits[0] if hits else None


def _run_child(code, env_extra, logdir):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", **env_extra)
    env["ASAN_OPTIONS"] = f"detect_leaks=0:halt_on_error=1:log_path={logdir}/asan"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={logdir}/ubsan"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(open(f).read() for f in glob.glob(os.path.join(logdir, "*san*")))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:] + r.stderr[-3000:] + reports[:4000])
    return r


def test_library_host_code_under_sanitizers(tmp_path):
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc not found")
    runtime = _clang_asan_runtime()
    if runtime is None:
        pytest.skip("clang's AddressSanitizer runtime not found")
    lib = str(tmp_path / "libdllm.so")
    cmd = ["hipcc", "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-shared", "-std=c++17", "-fno-honor-nans",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan",
           "-I", os.path.join(ROOT, "include"), "-o", lib, *sorted(glob.glob(os.path.join(CSRC, "*.hip")))]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    code = ("import sys, pytest\n"
            "from confidence_block_unmasking_amd import _lib\n"
            f"_lib.LIB_PATH = {lib!r}\n"
            "rc = pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi.py'])\n"
            f"assert _lib._lib is not None and _lib._lib._name == {lib!r}, 'the sanitized copy was not the one used'\n"
            "sys.exit(rc)\n")
    r = _run_child(code, {"LD_PRELOAD": runtime}, str(tmp_path))
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]


def test_generator_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    rts = [subprocess.run([gcc, f"-print-file-name={n}"], capture_output=True, text=True).stdout.strip()
           for n in ("libasan.so", "libubsan.so")]
    if not all(os.path.isabs(p) and os.path.exists(p) for p in rts):
        pytest.skip("gcc's sanitizer runtimes not found")
    lib = str(tmp_path / "libsynth_cpu.so")
    subprocess.run([gcc, "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared", "-fopenmp",
                    "-fsanitize=address,undefined", "-o", lib, os.path.join(ROOT, "workload", "synth.c")],
                   check=True, capture_output=True, timeout=300)
    code = ("import sys, pytest\n"
            "from workload import synth\n"
            f"synth.CPU_LIB = {lib!r}\n"
            "rc = pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', 'tests/test_workload.py'])\n"
            f"assert synth._cpu is not None and synth._cpu._name == {lib!r}, 'the sanitized copy was not the one used'\n"
            "sys.exit(rc)\n")
    r = _run_child(code, {"LD_PRELOAD": " ".join(rts)}, str(tmp_path))
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]
