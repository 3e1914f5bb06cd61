"""ctypes binding of ``libdsv4_attn.so`` (the C ABI in include/dsv4_attn.h).

Argument marshalling only: torch tensors become ``dsv4_tensor`` descriptors
(data pointer, dtype, shape, strides) and the current HIP stream handle is
passed through.  Every step of the attention runs in the HIP library; there is
no fallback, and loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# DSV4_ATTN_LIB may name another build of the same library (for example one
# whose host code carries sanitizers); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("DSV4_ATTN_LIB") or os.path.join(HERE, "libdsv4_attn.so")

DSV4_BF16, DSV4_F32, DSV4_I32, DSV4_U8 = 1, 2, 3, 4
STATUS = {0: "OK", 1: "ERR_INVALID", 2: "ERR_UNSUPPORTED", 3: "ERR_WORKSPACE", 4: "ERR_HIP", 5: "ERR_CONTRACT"}
_DTYPES = {torch.bfloat16: DSV4_BF16, torch.float32: DSV4_F32, torch.int32: DSV4_I32, torch.uint8: DSV4_U8}


class Dsv4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class Tensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


_lib = None
_lock = threading.Lock()


def load() -> ctypes.CDLL:
    """Load the HIP library (raises if it is missing: there is no fallback)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first (python -m hybrid_sparse_mqa_amd.build)"
            )
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Tensor)
        L.dsv4_attn_forward.restype = ctypes.c_int
        L.dsv4_attn_forward.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                        P, P, ctypes.c_void_p]
        L.dsv4_attn_forward_noalloc.restype = ctypes.c_int
        L.dsv4_attn_forward_noalloc.argtypes = L.dsv4_attn_forward.argtypes
        L.dsv4_attn_noalloc_scratch_bytes.restype = ctypes.c_size_t
        L.dsv4_attn_gather_slots.restype = ctypes.c_int
        L.dsv4_attn_gather_slots.argtypes = [P, P, P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P,
                                             ctypes.c_void_p]
        L.dsv4_c4_topk.restype = ctypes.c_int
        L.dsv4_c4_topk.argtypes = [P, P, P, ctypes.c_void_p]
        L.dsv4_kv_pack_fp8.restype = ctypes.c_int
        L.dsv4_kv_pack_fp8.argtypes = [P, P, P, ctypes.c_void_p]
        L.dsv4_last_error.restype = ctypes.c_char_p
        L.dsv4_abi_version.restype = ctypes.c_int32
        L.dsv4_attn_workspace_reserve.restype = ctypes.c_int
        L.dsv4_attn_workspace_reserve.argtypes = [ctypes.c_size_t, ctypes.c_void_p]
        L.dsv4_attn_workspace_release.restype = None
        L.dsv4_attn_set_split_keys.restype = ctypes.c_int
        L.dsv4_attn_set_split_keys.argtypes = [ctypes.c_int32]
        L.dsv4_attn_set_kernel.restype = ctypes.c_int
        L.dsv4_attn_set_kernel.argtypes = [ctypes.c_int32]
        L.dsv4_attn_plan.restype = ctypes.c_int
        L.dsv4_attn_plan.argtypes = [ctypes.c_int32] * 7 + [ctypes.POINTER(ctypes.c_int32)] * 3
        L.dsv4_attn_timing_enable.restype = ctypes.c_int
        L.dsv4_attn_timing_enable.argtypes = [ctypes.c_int32]
        L.dsv4_attn_timing_read.restype = ctypes.c_int
        L.dsv4_attn_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_int64)]
        L.dsv4_read_probe.restype = ctypes.c_int
        L.dsv4_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        L.dsv4_attn_debug_keys.restype = ctypes.c_int
        L.dsv4_attn_debug_keys.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64]
        _lib = L
        return L


def describe(t):
    """dsv4_tensor descriptor of a torch tensor (or None -> NULL)."""
    if t is None:
        return None
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() < 1 or t.dim() > 4:
        raise ValueError("descriptors hold 1..4 dimensions")
    d = Tensor()
    d.data = t.data_ptr() if t.numel() else (t.data_ptr() or 1)
    d.dtype = _DTYPES[t.dtype]
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def ref(d):
    return None if d is None else ctypes.byref(d)


def check(status: int):
    if status != 0:
        raise Dsv4Error(status, load().dsv4_last_error().decode())


def stream_handle(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream
