"""Python entry points with the names of the C ABI (include/dsv4_attn.h).

They only build descriptors and pass the current stream; all work happens in
``libdsv4_attn.so``.  Tensors must already be on the GPU.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _native as N


def dsv4_attn_forward(
    q: torch.Tensor,
    swa_pool: torch.Tensor,
    swa_page_table: torch.Tensor,
    extra_pool: Optional[torch.Tensor],
    extra_page_table: Optional[torch.Tensor],
    c4_indices: Optional[torch.Tensor],
    seq_lens: torch.Tensor,
    qo_indptr: torch.Tensor,
    sink: Optional[torch.Tensor],
    compress_ratio: int,
    window: int,
    scale: float,
    out: Optional[torch.Tensor] = None,
    lse: Optional[torch.Tensor] = None,
    return_lse: bool = True,
    stream: Optional[int] = None,
    noalloc: bool = False,
) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """SWA + (C4 | C128) attention of every query row; returns (out, lse).
    noalloc: call dsv4_attn_forward_noalloc instead."""
    L = N.load()
    T, H = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    descs = [N.describe(x) for x in (q, swa_pool, swa_page_table, extra_pool, extra_page_table, c4_indices,
                                     seq_lens, qo_indptr, sink, out, lse)]
    st = N.stream_handle(q.device) if stream is None else stream
    fn = L.dsv4_attn_forward_noalloc if noalloc else L.dsv4_attn_forward
    N.check(fn(*[N.ref(d) for d in descs[:9]], int(compress_ratio), int(window), float(scale),
               N.ref(descs[9]), N.ref(descs[10]), ctypes.c_void_p(st)))
    return out, lse


def dsv4_attn_forward_noalloc(*args, **kwargs) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """dsv4_attn_forward through the no-allocation entry point (pass ``out``
    and ``lse`` to allocate nothing here either)."""
    return dsv4_attn_forward(*args, noalloc=True, **kwargs)


def dsv4_attn_noalloc_scratch_bytes() -> int:
    return int(N.load().dsv4_attn_noalloc_scratch_bytes())


def dsv4_attn_gather_slots(
    swa_page_table: torch.Tensor,
    extra_page_table: Optional[torch.Tensor],
    c4_indices: Optional[torch.Tensor],
    seq_lens: torch.Tensor,
    qo_indptr: torch.Tensor,
    num_rows: int,
    compress_ratio: int,
    window: int,
    slots: Optional[torch.Tensor] = None,
    counts: Optional[torch.Tensor] = None,
    stream: Optional[int] = None,
) -> Tuple[torch.Tensor, torch.Tensor]:
    """Canonical slot list of every row (slots [T, Kmax], counts [T, 2])."""
    L = N.load()
    dev = swa_page_table.device
    if slots is None:
        extra = 0
        if compress_ratio == 4:
            extra = c4_indices.shape[1]
        elif compress_ratio == 128:
            extra = 256 * extra_page_table.shape[1]
        slots = torch.empty((num_rows, window + extra), dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty((num_rows, 2), dtype=torch.int32, device=dev)
    descs = [N.describe(x) for x in (swa_page_table, extra_page_table, c4_indices, seq_lens, qo_indptr, slots, counts)]
    st = N.stream_handle(dev) if stream is None else stream
    N.check(L.dsv4_attn_gather_slots(
        *[N.ref(d) for d in descs[:5]], int(num_rows), int(compress_ratio), int(window),
        N.ref(descs[5]), N.ref(descs[6]), ctypes.c_void_p(st)))
    return slots, counts


def dsv4_kv_pack_fp8(k: torch.Tensor, slots: torch.Tensor, pool: torch.Tensor, stream: Optional[int] = None) -> None:
    """Quantise K rows (bf16 [n, 512]) into the packed FP8 pool (uint8
    [pages, 149504], written in place) at ``slots`` (int32 [n], < 0 skips)."""
    L = N.load()
    descs = [N.describe(x) for x in (k, slots, pool)]
    st = N.stream_handle(k.device) if stream is None else stream
    N.check(L.dsv4_kv_pack_fp8(*[N.ref(d) for d in descs], ctypes.c_void_p(st)))


def dsv4_c4_topk(scores: torch.Tensor, num_candidates: torch.Tensor, k: int = 512,
                 indices: Optional[torch.Tensor] = None, stream: Optional[int] = None) -> torch.Tensor:
    """Per row, the k highest of scores[t, :num_candidates[t]] (ties: the lower
    index), ascending, then -1: int32 [T, k], the C4 index lists."""
    L = N.load()
    if indices is None:
        indices = torch.empty((scores.shape[0], k), dtype=torch.int32, device=scores.device)
    descs = [N.describe(x) for x in (scores, num_candidates, indices)]
    st = N.stream_handle(scores.device) if stream is None else stream
    N.check(L.dsv4_c4_topk(*[N.ref(d) for d in descs], ctypes.c_void_p(st)))
    return indices


def dsv4_abi_version() -> int:
    return int(N.load().dsv4_abi_version())


def dsv4_last_error() -> str:
    return N.load().dsv4_last_error().decode()


def dsv4_attn_set_split_keys(keys_per_split: int) -> None:
    N.check(N.load().dsv4_attn_set_split_keys(int(keys_per_split)))


# Split-kernel variants (DSV4_KERNEL_* in dsv4_attn.h) and their heads per workgroup.
KERNEL_AUTO, KERNEL_H16, KERNEL_H32, KERNEL_H32_ROLES, KERNEL_H64, KERNEL_FP8 = range(6)
KERNEL_HEADS = {KERNEL_H16: 16, KERNEL_H32: 32, KERNEL_H32_ROLES: 32, KERNEL_H64: 64, KERNEL_FP8: 64}


def dsv4_attn_set_kernel(kernel: int) -> None:
    N.check(N.load().dsv4_attn_set_kernel(int(kernel)))


def dsv4_attn_plan(num_rows, num_heads, compress_ratio, window, c4_width=0, extra_pages=0,
                   kv_fp8=False) -> Tuple[int, int, int]:
    """(splits per row and head block, keys per split, split-kernel variant)
    that dsv4_attn_forward would use."""
    s = ctypes.c_int32()
    c = ctypes.c_int32()
    k = ctypes.c_int32()
    N.check(N.load().dsv4_attn_plan(int(num_rows), int(num_heads), int(compress_ratio), int(window), int(c4_width),
                                    int(extra_pages), int(bool(kv_fp8)), ctypes.byref(s), ctypes.byref(c),
                                    ctypes.byref(k)))
    return s.value, c.value, k.value


def dsv4_attn_workspace_reserve(nbytes: int, stream: Optional[int] = None) -> None:
    st = N.stream_handle() if stream is None else stream
    N.check(N.load().dsv4_attn_workspace_reserve(int(nbytes), ctypes.c_void_p(st)))


def dsv4_attn_workspace_release() -> None:
    N.load().dsv4_attn_workspace_release()


def dsv4_attn_debug_keys(keys: Optional[torch.Tensor], masks: Optional[torch.Tensor] = None) -> None:
    """Test hook: while ``keys`` (int64, device) is given, forward calls run the
    recording builds of the split kernels (see dsv4_attn.h); None stops it."""
    if keys is None:
        N.check(N.load().dsv4_attn_debug_keys(None, 0, None, 0))
        return
    N.check(N.load().dsv4_attn_debug_keys(ctypes.c_void_p(keys.data_ptr()), keys.numel(),
                                          ctypes.c_void_p(masks.data_ptr()), masks.numel()))


def dsv4_attn_timing_enable(enable: bool) -> None:
    N.check(N.load().dsv4_attn_timing_enable(int(bool(enable))))


def dsv4_attn_timing_read() -> Tuple[float, float, int]:
    """(summed split-kernel ms, summed merge-kernel ms, calls) recorded since the last read."""
    a = ctypes.c_double()
    b = ctypes.c_double()
    n = ctypes.c_int64()
    N.check(N.load().dsv4_attn_timing_read(ctypes.byref(a), ctypes.byref(b), ctypes.byref(n)))
    return a.value, b.value, n.value


def dsv4_read_probe(buf: torch.Tensor, nbytes: int, workgroups: int, sink: torch.Tensor,
                    stream: Optional[int] = None) -> None:
    """Plain streaming read of the first ``nbytes`` bytes of ``buf`` (timing helper)."""
    if nbytes > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    if sink.numel() * sink.element_size() < 16:
        raise ValueError("sink must hold 16 bytes")
    N.check(N.load().dsv4_read_probe(ctypes.c_void_p(buf.data_ptr()), int(nbytes), int(workgroups),
                                     ctypes.c_void_p(sink.data_ptr()),
                                     ctypes.c_void_p(N.stream_handle(buf.device) if stream is None else stream)))

