"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two instrumented builds, each exercised in a child Python that preloads its
sanitizer runtime (any report fails the child, and so the test):

* the C-ABI host code: ``dsv4_api.cpp`` recompiled with the sanitizers on its
  host side only (device code is never instrumented) and linked with the
  library's existing kernel objects; the child runs ``tests/test_abi_host.py``
  (symbol exports and every argument error, no GPU needed);
* the oracle: ``oracle/dsv4_oracle.c`` built by gcc with the sanitizers; the
  child runs the oracle's pins (brute force, closed forms, tables, packer,
  top-k) without the mutant builds.

The two use different sanitizer runtimes (clang's for the library, gcc's for
the oracle), so they run in separate children.
"""
import glob
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "hybrid_sparse_mqa_amd", "csrc")
KERNEL_OBJS = [os.path.join(CSRC, f + ".o") for f in ("dsv4_attn_kernels.hip", "dsv4_pack.hip", "dsv4_topk.hip", "dsv4_probe.hip")]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-6000:]}"
    return r.stdout


def _child_env(extra):
    env = dict(os.environ)
    env.update(extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    return env


def test_abi_host_code_under_asan_ubsan(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    runtime = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                            "libclang_rt.asan-x86_64.so")))
    if not os.path.exists(hipcc) or not runtime or not all(map(os.path.exists, KERNEL_OBJS)):
        pytest.skip("needs hipcc, clang's ASan runtime and a built HIP library")
    obj = str(tmp_path / "dsv4_api_san.o")
    lib = str(tmp_path / "libdsv4_attn_san.so")
    host_san = [
        "-Xarch_host", "-fsanitize=address",
        "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-sanitize-recover=all",
        "-Xarch_host", "-fno-omit-frame-pointer",
    ]
    _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), *host_san,
          "-x", "hip", "-c", os.path.join(CSRC, "dsv4_api.cpp"), "-o", obj])
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *host_san[:4],
          "-Xarch_host", "-shared-libasan", *KERNEL_OBJS, obj, "-o", lib])
    out = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                os.path.join(HERE, "test_abi_host.py")], cwd=ROOT, timeout=600,
               env=_child_env({"DSV4_ATTN_LIB": lib, "LD_PRELOAD": runtime[-1]}))
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out


def test_oracle_under_asan_ubsan(tmp_path):
    try:
        asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True,
                              check=True).stdout.strip()
        ubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], stdout=subprocess.PIPE, text=True,
                               check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        pytest.skip("gcc not available")
    if not (os.path.isabs(asan) and os.path.isabs(ubsan)):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    lib = str(tmp_path / "libdsv4_oracle_san.so")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          os.path.join(ROOT, "oracle", "dsv4_oracle.c"), "-o", lib, "-lm"])
    tests = [os.path.join(HERE, f) for f in ("test_oracle_pins.py", "test_oracle_pack.py", "test_oracle_topk.py")]
    out = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                "-k", "not mutant", *tests], cwd=ROOT, timeout=900,
               env=_child_env({"DSV4O_LIB": lib, "LD_PRELOAD": f"{asan} {ubsan}", "OMP_NUM_THREADS": "4"}))
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
