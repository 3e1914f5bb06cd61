"""DeepSeek-V4 hybrid sparse MQA attention (decode / target-verify) on MI355X.

The compute path is the HIP library ``libdsv4_attn.so`` (hand-written gfx950
kernels behind the C ABI in include/dsv4_attn.h); this package is its Python
binding.  Importing the package does not load the library; the first call
does, and raises if it has not been built.
"""
from .api import (  # noqa: F401
    dsv4_abi_version,
    dsv4_attn_debug_keys,
    dsv4_attn_forward,
    dsv4_attn_forward_noalloc,
    dsv4_attn_noalloc_scratch_bytes,
    dsv4_attn_gather_slots,
    dsv4_kv_pack_fp8,
    dsv4_c4_topk,
    dsv4_attn_plan,
    dsv4_attn_set_kernel,
    dsv4_attn_set_split_keys,
    dsv4_attn_timing_enable,
    dsv4_attn_timing_read,
    dsv4_attn_workspace_release,
    dsv4_attn_workspace_reserve,
    dsv4_last_error,
    dsv4_read_probe,
)
from ._native import Dsv4Error, LIB_PATH  # noqa: F401
