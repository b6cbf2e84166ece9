"""Compile check_c_abi (a plain C caller of the library's C ABI, checked
against the CPU oracle) next to this file.  Test infrastructure: linked
against the in-tree librws_softmax.so and the oracle's C sources."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BINARY = os.path.join(HERE, "check_c_abi")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    lib_dir = os.path.join(ROOT, "row_wise_safe_amd")
    tmp = BINARY + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-ffp-contract=off",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(HERE, "check_c_abi.c"),
           os.path.join(ROOT, "oracle", "softmax_oracle.c"),
           os.path.join(ROOT, "oracle", "norm_oracle.c"),
           f"-L{lib_dir}", "-lrws_softmax", f"-L{ROCM}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../row_wise_safe_amd", f"-Wl,-rpath,{ROCM}/lib",
           "-lm", "-lpthread", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, BINARY)
    return BINARY


if __name__ == "__main__":
    print(build(verbose=True))
