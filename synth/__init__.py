"""Seeded synthetic inputs for DeepSeek-V4 hybrid sparse MQA attention.

This package only draws random numbers and lays them out in memory: query
rows, paged SWA and compressed KV pools, page tables, C4 index lists and sink
logits.  It holds none of the attention arithmetic (no gather, no softmax, no
FP8 decode), so both the CPU oracle and the HIP path can take their inputs
from here without sharing any of the method's code.
"""
from .workloads import (  # noqa: F401
    Case,
    CONFIGS,
    D_HEAD,
    D_NOPE,
    D_ROPE,
    FP8_PAGE_BYTES,
    FP8_ROW_BYTES,
    FP8_SCALE_OFFSET,
    PAGE_SIZE,
    make_case,
    make_config,
    quantize_fp8_rows,
    store_float_rows,
    tile_requests,
)
