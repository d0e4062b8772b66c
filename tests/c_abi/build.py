"""Build tests/c_abi/step_consumer: a C program that uses libdit_attn.so through
include/dit_attn.h only (hipMalloc'd buffers, its own stream), for the C-ABI tests.

    python tests/c_abi/build.py
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "partitioned_state_reuse_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
BIN = os.path.join(HERE, "step_consumer")


def build(verbose: bool = False) -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler")
    # the HIP runtime header selects the AMD implementation through this macro (hipcc sets it
    # itself; a plain C compiler needs it on the command line)
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "step_consumer.c"),
           "-L", PKG, "-ldit_attn", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../partitioned_state_reuse_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", BIN + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
