"""fp64 CPU oracle for DeepSeek-V4 hybrid sparse MQA attention.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg use it to check the HIP library.  The product path never
imports, loads or calls anything here.  The arithmetic lives in
``dsv4_oracle.c`` (plain C, fp64, OpenMP over rows); this module compiles it
with gcc and wraps it with ctypes.

Parity status: every function is pinned by ``tests/test_oracle_pins.py``
(brute force over unpaged logical rows, closed forms, invariants, the worked
examples of the DSV4 walk-through page, the E4M3FN code table and mutants);
the FP8 packer by ``tests/test_oracle_pack.py`` (torch's float8_e4m3fn
conversion, round-trip error bounds, closed forms, the byte layout, mutants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dsv4_oracle.c")


def lib_path(mutant: int = 0, out_dir: Optional[str] = None) -> str:
    name = "libdsv4_oracle.so" if mutant == 0 else f"libdsv4_oracle_m{mutant}.so"
    return os.path.join(out_dir or HERE, name)


def build(mutant: int = 0, out_dir: Optional[str] = None) -> str:
    """Compile the oracle (or one of its deliberately wrong variants)."""
    out = lib_path(mutant, out_dir)
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra",
           f"-DDSV4O_MUTANT={int(mutant)}", SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class _Case(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("W", ctypes.c_int32), ("R", ctypes.c_int32), ("kv_fp8", ctypes.c_int32),
        ("seq_lens", ctypes.c_void_p), ("qo_indptr", ctypes.c_void_p),
        ("q", ctypes.c_void_p), ("sink", ctypes.c_void_p),
        ("swa_pool", ctypes.c_void_p), ("swa_pool_pages", ctypes.c_int64),
        ("swa_page_table", ctypes.c_void_p), ("p_swa", ctypes.c_int32),
        ("extra_pool", ctypes.c_void_p), ("extra_pool_pages", ctypes.c_int64),
        ("extra_page_table", ctypes.c_void_p), ("p_extra", ctypes.c_int32),
        ("c4_indices", ctypes.c_void_p), ("K", ctypes.c_int32),
        ("scale", ctypes.c_double),
    ]


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data


class Oracle:
    """ctypes handle on one compiled oracle library."""

    def __init__(self, path: Optional[str] = None, mutant: int = 0):
        if path is None and mutant == 0 and os.environ.get("DSV4O_LIB"):
            path = os.environ["DSV4O_LIB"]  # another build of the same source (e.g. with sanitizers)
        if path is None:
            path = lib_path(mutant)
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
                build(mutant)
        self.lib = ctypes.CDLL(path)
        L = self.lib
        L.dsv4o_gather.restype = ctypes.c_int
        L.dsv4o_gather.argtypes = [ctypes.POINTER(_Case), ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.dsv4o_attention.restype = ctypes.c_int
        L.dsv4o_attention.argtypes = [ctypes.POINTER(_Case), ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
        L.dsv4o_last_error.restype = ctypes.c_char_p
        L.dsv4o_bf16_to_double.restype = ctypes.c_double
        L.dsv4o_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.dsv4o_e4m3_to_double.restype = ctypes.c_double
        L.dsv4o_e4m3_to_double.argtypes = [ctypes.c_uint8]
        L.dsv4o_e4m3_from_float.restype = ctypes.c_uint8
        L.dsv4o_e4m3_from_float.argtypes = [ctypes.c_float]
        L.dsv4o_pack_fp8.restype = ctypes.c_int
        L.dsv4o_pack_fp8.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64]
        L.dsv4o_max_threads.restype = ctypes.c_int
        L.dsv4o_mutant.restype = ctypes.c_int

    # ------------------------------------------------------------------
    def _struct(self, case):
        keep = []

        def arr(a, dt):
            if a is None:
                return None
            a = np.ascontiguousarray(a, dtype=dt)
            keep.append(a)
            return a

        fp8 = case.kv == "fp8"
        swa = arr(case.swa_pool, case.swa_pool.dtype)
        ext = arr(case.extra_pool, None if case.extra_pool is None else case.extra_pool.dtype)
        pages = lambda pool: 0 if pool is None else (pool.shape[0] if fp8 else pool.shape[0] // 256)
        st = _Case(
            B=case.B, T=case.T, H=case.H, W=case.W, R=case.R, kv_fp8=int(fp8),
            seq_lens=_ptr(arr(case.seq_lens, np.int32)),
            qo_indptr=_ptr(arr(case.qo_indptr, np.int32)),
            q=_ptr(arr(case.q, np.uint16)),
            sink=_ptr(arr(case.sink, np.float32)),
            swa_pool=_ptr(swa), swa_pool_pages=pages(swa),
            swa_page_table=_ptr(arr(case.swa_page_table, np.int32)),
            p_swa=case.swa_page_table.shape[1],
            extra_pool=_ptr(ext), extra_pool_pages=pages(ext),
            extra_page_table=_ptr(arr(case.extra_page_table, np.int32)),
            p_extra=0 if case.extra_page_table is None else case.extra_page_table.shape[1],
            c4_indices=_ptr(arr(case.c4_indices, np.int32)),
            K=case.K, scale=case.scale,
        )
        return st, keep

    def _err(self):
        return OracleError(self.lib.dsv4o_last_error().decode())

    def gather(self, case, t: int):
        """(swa_slots, extra_slots) of row t in canonical order (int32 arrays)."""
        st, keep = self._struct(case)
        p_extra = 0 if case.extra_page_table is None else case.extra_page_table.shape[1]
        swa = np.zeros(case.W + 1, np.int32)
        ext = np.zeros(max(case.K, p_extra * 256, 1), np.int32)
        ns = np.zeros(1, np.int32)
        ne = np.zeros(1, np.int32)
        rc = self.lib.dsv4o_gather(ctypes.byref(st), int(t), _ptr(swa), _ptr(ns), _ptr(ext), _ptr(ne))
        if rc:
            raise self._err()
        return swa[: ns[0]].copy(), ext[: ne[0]].copy()

    def attention(self, case, rows=None, nthreads: int = 0):
        """fp64 (out [n,H,512], lse [n,H], lse_nosink [n,H]) for the given rows."""
        st, keep = self._struct(case)
        rows = np.arange(case.T, dtype=np.int32) if rows is None else np.asarray(rows, dtype=np.int32)
        n = len(rows)
        out = np.zeros((n, case.H, 512), np.float64)
        lse = np.zeros((n, case.H), np.float64)
        lse_ns = np.zeros((n, case.H), np.float64)
        if n:
            rc = self.lib.dsv4o_attention(ctypes.byref(st), _ptr(rows), n, _ptr(out), _ptr(lse), _ptr(lse_ns),
                                          int(nthreads))
            if rc:
                raise self._err()
        return out, lse, lse_ns

    def pack_fp8(self, k_bits: np.ndarray, slots: np.ndarray, pool: np.ndarray) -> None:
        """Quantise K rows (bf16 bits [n, 512]) into packed FP8 records of
        ``pool`` (uint8 [pages, 149504], modified in place) at ``slots``."""
        k_bits = np.ascontiguousarray(k_bits, dtype=np.uint16)
        slots = np.ascontiguousarray(slots, dtype=np.int32)
        assert k_bits.ndim == 2 and k_bits.shape[1] == 512 and slots.shape == (k_bits.shape[0],)
        assert pool.dtype == np.uint8 and pool.flags.c_contiguous and pool.ndim == 2
        rc = self.lib.dsv4o_pack_fp8(_ptr(k_bits), _ptr(slots), int(k_bits.shape[0]), _ptr(pool), int(pool.shape[0]))
        if rc:
            raise self._err()

    def e4m3_from_float(self, x: float) -> int:
        return int(self.lib.dsv4o_e4m3_from_float(ctypes.c_float(x)))

    def bf16_to_double(self, bits: int) -> float:
        return self.lib.dsv4o_bf16_to_double(bits)

    def e4m3_to_double(self, code: int) -> float:
        return self.lib.dsv4o_e4m3_to_double(code)

    def max_threads(self) -> int:
        return self.lib.dsv4o_max_threads()
