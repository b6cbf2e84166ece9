"""Build librws_softmax.so (the gfx950 HIP kernels and the C ABI) in-tree.

hipcc cross-compiles for gfx950 without a GPU.  Every translation unit is
compiled with packed-fp32 instruction generation disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIBRARY = os.path.join(HERE, "librws_softmax.so")
ARCH = "gfx950"

SOURCES = [
    "rws_api.cpp",
    "rws_wave_row.hip",
    "rws_tile_rows.hip",
    "rws_block_onepass.hip",
    "rws_two_pass.hip",
    "rws_splitk.hip",
    "rws_reference.hip",
    "rws_splitk_fused.hip",
    "rws_splitk_ordered.hip",
    "rws_masked.hip",
    "rws_backward.hip",
    "rws_norm_wave.hip",
    "rws_norm_block.hip",
]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _filter(out: str) -> str:
    # hipcc's host pass does not know the gfx950 feature flag; that note is noise.
    return "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source for gfx950 and link the shared library."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    procs = []
    objects = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objects.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [cc, *COMMON_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        msg = _filter(out)
        if msg.strip() and (verbose or p.returncode != 0):
            print(msg, file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for: {', '.join(failed)}")
    tmp = LIBRARY + f".tmp{os.getpid()}"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objects]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        print(_filter(r.stdout), file=sys.stderr)
        raise RuntimeError("linking librws_softmax.so failed")
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
