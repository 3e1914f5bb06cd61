"""Build step of the HIP library: ``libdsv4_attn.so`` for gfx950, in-tree.

Compiles the kernels and the C-ABI host code with hipcc.  Every HIP source is
built with packed-FP32 instruction forms disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdsv4_attn.so")
SOURCES = ["dsv4_attn_kernels.hip", "dsv4_pack.hip", "dsv4_topk.hip", "dsv4_probe.hip", "dsv4_api.cpp"]
ARCH = os.environ.get("DSV4_OFFLOAD_ARCH", "gfx950")
# Per-source flags.  The top-k kernels issue their list-offset atomic from one
# thread and use its result later; the compiler's atomic combining (a wave
# reduction around a uniform-address atomic) would wait for the result at once.
EXTRA_FLAGS = {"dsv4_topk.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the HIP library)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


def _compile(src: str, verbose: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(CSRC, src + ".o")
    cmd = [hipcc(), *compile_flags(), *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}")
    if verbose and r.stdout:
        print(r.stdout, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source (in parallel) and link the shared library;
    returns its path."""
    from concurrent.futures import ThreadPoolExecutor

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
