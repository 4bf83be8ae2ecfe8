"""Build tests/c/step_from_c (a C program that calls dllm_step through the C ABI with the HIP
runtime API alone) with gcc, against the in-tree libdllm.so.  Test infrastructure: run by
__graft_entry__.build(); the GPU test tests/test_gpu_c_program.py runs the result."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "step_from_c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose=False):
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "step_from_c.c"), "-o", EXE + ".tmp",
           "-L", os.path.join(ROOT, "confidence_block_unmasking_amd"), "-ldllm",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../confidence_block_unmasking_amd", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
