"""Seeded synthetic workloads shaped like the DeepSeek-V4 attention tests and
the decode / target-verify configurations of the hybrid sparse MQA path.

Everything here is input construction: random draws (numpy PCG64), casts to
the storage formats (bf16 and OCP FP8 E4M3 through torch's own conversions),
and the placement of rows into paged pools through shuffled page tables.  No
attention arithmetic lives here.

Storage formats (the SGLang DSV4 test-matrix page, "packed FP8 nope + BF16
rope", 584 bytes per token; our record layout is a choice of this library):

* bf16 pool: ``uint16 [num_pages * 256, 512]``; slot ``s`` is row ``s``.
* fp8 pool: ``uint8 [num_pages, 149504]``.  A page holds 256 records of 576
  bytes ``[448 x e4m3 nope | 64 x bf16 rope]``, then 256 fp32 per-token scales,
  then 1 KiB of padding: 256 x 584 bytes, every record 16-byte aligned.
  Slot ``s`` lives in page ``s // 256`` at record ``s % 256``.

Positions follow the DSV4 attention walk-through ("Query, cache write and
history addressing", section 1): a request of total length ``L`` whose pass
holds ``n_q`` query rows places them at positions ``L - n_q .. L - 1``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

PAGE_SIZE = 256
D_HEAD = 512
D_NOPE = 448
D_ROPE = 64
FP8_ROW_BYTES = D_NOPE + 2 * D_ROPE            # 576
FP8_SCALE_OFFSET = PAGE_SIZE * FP8_ROW_BYTES   # 147456
FP8_PAGE_BYTES = PAGE_SIZE * 584               # 149504

POISON_BYTE = 0xFF  # NaN as bf16 (0xFFFF), as e4m3 (0xFF) and as fp32


@dataclass
class Case:
    """One batch of inputs for a single attention call (host numpy arrays)."""

    name: str
    H: int
    W: int
    R: int
    kv: str                       # "bf16" or "fp8"
    scale: float
    seq_lens: np.ndarray          # int32 [B]
    qo_indptr: np.ndarray         # int32 [B+1]
    q: np.ndarray                 # uint16 (bf16 bits) [T, H, 512]
    sink: Optional[np.ndarray]    # float32 [H] or None
    swa_pool: np.ndarray          # bf16: uint16 [S, 512]; fp8: uint8 [pages, 149504]
    swa_page_table: np.ndarray    # int32 [B, P_swa]
    extra_pool: Optional[np.ndarray]
    extra_page_table: Optional[np.ndarray]
    c4_indices: Optional[np.ndarray]   # int32 [T, K], -1 padded
    poison_swa_page: int = -1
    poison_extra_page: int = -1
    # Logical (unpaged) rows, kept for small cases only.  Per request:
    #   "tok_lo": first live token position; "tok": rows of tokens tok_lo..L-1
    #   "cmp_ids": compressed entry ids holding data; "cmp": their rows.
    # Rows are uint16 [n, 512] (bf16) or a tuple (codes u8 [n,448],
    # scales f32 [n], rope u16 [n,64]) (fp8).
    logical: Optional[List[Dict]] = None
    meta: Dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def T(self) -> int:
        return int(self.qo_indptr[-1])

    @property
    def K(self) -> int:
        return 0 if self.c4_indices is None else int(self.c4_indices.shape[1])


# --------------------------------------------------------------------------
# Storage-format casts (library conversions only)
# --------------------------------------------------------------------------
def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).clamp_(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quantize_fp8_rows(nope: np.ndarray, rope_bits: np.ndarray):
    """Packed-FP8 storage of float32 non-rotary dims [n, 448] and bf16 rotary
    bits [n, 64]: per-token scale amax/448 (1 for an all-zero row) and the
    E4M3FN codes of nope/scale through torch's conversion."""
    nope = np.ascontiguousarray(nope, dtype=np.float32)
    n = nope.shape[0]
    amax = np.abs(nope).max(axis=1) if n else np.zeros(0, np.float32)
    scales = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = _to_e4m3_codes(nope / scales[:, None])
    return (codes, scales, np.ascontiguousarray(rope_bits, dtype=np.uint16))


def _draw_rows(rng: np.random.Generator, n: int, kv: str):
    """Draw ``n`` KV rows ~ N(0,1) in the pool's storage format."""
    if kv == "bf16":
        return _to_bf16_bits(rng.standard_normal((n, D_HEAD), dtype=np.float32))
    nope = rng.standard_normal((n, D_NOPE), dtype=np.float32)
    rope = _to_bf16_bits(rng.standard_normal((n, D_ROPE), dtype=np.float32))
    return quantize_fp8_rows(nope, rope)


def store_float_rows(pool: np.ndarray, kv: str, slots, rows_f32: np.ndarray) -> None:
    """Write float32 rows [n, 512] at physical slots, cast to the pool's
    storage format (bf16, or packed FP8 via quantize_fp8_rows)."""
    slots = np.asarray(slots, dtype=np.int64).reshape(-1)
    rows_f32 = np.asarray(rows_f32, dtype=np.float32).reshape(len(slots), D_HEAD)
    if kv == "bf16":
        _store_rows(pool, kv, slots, _to_bf16_bits(rows_f32))
    else:
        _store_rows(pool, kv, slots, quantize_fp8_rows(rows_f32[:, :D_NOPE], _to_bf16_bits(rows_f32[:, D_NOPE:])))


def _rows_take(rows, sel):
    if isinstance(rows, tuple):
        return tuple(r[sel] for r in rows)
    return rows[sel]


def _alloc_pool(num_pages: int, kv: str) -> np.ndarray:
    if kv == "bf16":
        return np.full((num_pages * PAGE_SIZE, D_HEAD), 0xFFFF, dtype=np.uint16)
    return np.full((num_pages, FP8_PAGE_BYTES), POISON_BYTE, dtype=np.uint8)


def _store_rows(pool: np.ndarray, kv: str, slots: np.ndarray, rows) -> None:
    """Write rows into the pool at physical slots (the store side of the cache)."""
    if len(slots) == 0:
        return
    if kv == "bf16":
        pool[slots] = rows
        return
    codes, scales, rope = rows
    page = slots // PAGE_SIZE
    rec = slots % PAGE_SIZE
    base = rec * FP8_ROW_BYTES
    cols = np.arange(D_NOPE)
    pool[page[:, None], base[:, None] + cols[None, :]] = codes
    rope_bytes = np.ascontiguousarray(rope).view(np.uint8).reshape(len(slots), 2 * D_ROPE)
    cols = np.arange(2 * D_ROPE)
    pool[page[:, None], base[:, None] + D_NOPE + cols[None, :]] = rope_bytes
    sc_bytes = np.ascontiguousarray(scales, dtype=np.float32).view(np.uint8).reshape(len(slots), 4)
    cols = np.arange(4)
    pool[page[:, None], FP8_SCALE_OFFSET + 4 * rec[:, None] + cols[None, :]] = sc_bytes


# --------------------------------------------------------------------------
# Case construction
# --------------------------------------------------------------------------
def make_case(
    *,
    seq_lens,
    n_q,
    H: int,
    R: int,
    W: int = 128,
    K: int = 512,
    kv: str = "bf16",
    sink: bool = True,
    sink_value: Optional[float] = None,
    seed: int = 0,
    n_sel: Optional[int] = None,
    pad_mode: str = "tail",
    decoy_frac: float = 0.125,
    keep_logical: bool = False,
    scale: Optional[float] = None,
    index_sets: int = 1,
    name: str = "case",
) -> Case:
    """Build one seeded batch.

    ``seq_lens[r]`` is the total length of request ``r`` including its
    ``n_q[r]`` query rows.  ``R`` is the compress ratio (0, 4 or 128).  For
    ``R == 4`` every row gets ``min(n_sel or K, visible)`` unique indices drawn
    from its visible compressed positions ``[0, (p+1)//4)``, then ``-1``
    padding to width ``K`` (``pad_mode`` "tail" or "scatter").
    Draw order: q, sink, per-request token rows, compressed rows, indices,
    page permutations.

    ``index_sets > 1`` (R == 4, benchmark rotation): ``index_sets - 1`` more
    index lists per row, each drawn like the first from a second generator,
    are stored in ``meta["c4_sets"]`` ([index_sets, T, K], set 0 being
    ``c4_indices``), and every entry any of them names is backed.
    """
    if R not in (0, 4, 128):
        raise ValueError(f"compress ratio {R}")
    if kv not in ("bf16", "fp8"):
        raise ValueError(kv)
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = len(seq_lens)
    n_q = np.broadcast_to(np.asarray(n_q, dtype=np.int64), (B,)).copy()
    if np.any(n_q < 0) or np.any(n_q > seq_lens):
        raise ValueError("need 0 <= n_q <= seq_len")
    qo_indptr = np.zeros(B + 1, dtype=np.int64)
    qo_indptr[1:] = np.cumsum(n_q)
    T = int(qo_indptr[-1])
    if scale is None:
        scale = float(D_HEAD) ** -0.5

    q = _to_bf16_bits(rng.standard_normal((T, H, D_HEAD), dtype=np.float32))
    sink_arr = None
    if sink:
        if sink_value is not None:
            sink_arr = np.full(H, sink_value, dtype=np.float32)
        else:
            sink_arr = rng.standard_normal(H, dtype=np.float32)

    # Row positions: the last n_q positions of each request.
    row_req = np.repeat(np.arange(B), n_q)
    row_pos = np.concatenate(
        [np.arange(seq_lens[r] - n_q[r], seq_lens[r]) for r in range(B)] or [np.zeros(0, np.int64)]
    ).astype(np.int64)

    # ---- live token rows (only the window of this pass's rows is kept) ----
    tok_lo = np.maximum(0, seq_lens - n_q - W + 1)
    tok_rows = [_draw_rows(rng, int(seq_lens[r] - tok_lo[r]), kv) for r in range(B)]

    # ---- compressed entries ----
    n_ent = seq_lens // R if R else np.zeros(B, np.int64)
    cmp_ids: List[np.ndarray] = []
    cmp_rows = []
    c4 = None
    if R == 128:
        for r in range(B):
            ids = np.arange(n_ent[r])
            cmp_ids.append(ids)
            cmp_rows.append(_draw_rows(rng, len(ids), kv))
    elif R == 4:
        c4 = np.full((T, K), -1, dtype=np.int64)
        want = K if n_sel is None else n_sel
        for t in range(T):
            vis = int((row_pos[t] + 1) // 4)
            m = min(want, vis, K)
            sel = rng.choice(vis, size=m, replace=False) if m else np.zeros(0, np.int64)
            if pad_mode == "scatter":
                where = np.sort(rng.choice(K, size=m, replace=False))
                c4[t, where] = sel
            else:
                c4[t, :m] = sel
        c4_sets = [c4]
        if index_sets > 1:
            rng_sets = np.random.Generator(np.random.PCG64(seed + 104729))
            for _ in range(index_sets - 1):
                extra = np.full((T, K), -1, dtype=np.int64)
                for t in range(T):
                    vis = int((row_pos[t] + 1) // 4)
                    m = min(want, vis, K)
                    extra[t, :m] = rng_sets.choice(vis, size=m, replace=False) if m else np.zeros(0, np.int64)
                c4_sets.append(extra)
        for r in range(B):
            rows_r = np.concatenate([cs[qo_indptr[r]:qo_indptr[r + 1]].reshape(-1) for cs in c4_sets])
            ids = np.unique(rows_r[rows_r >= 0])
            cmp_ids.append(ids)
            cmp_rows.append(_draw_rows(rng, len(ids), kv))

    # ---- SWA pages: only the pages holding live tokens are backed ----
    swa_pages_per_req = [
        list(range(int(tok_lo[r]) // PAGE_SIZE, (int(seq_lens[r]) - 1) // PAGE_SIZE + 1)) if seq_lens[r] > 0 else []
        for r in range(B)
    ]
    n_live = sum(len(p) for p in swa_pages_per_req)
    n_pages = n_live + max(1, int(round(decoy_frac * n_live))) + 1
    perm = rng.permutation(n_pages)
    poison_swa = int(perm[-1])
    P_swa = max(1, int(max((int(L) + PAGE_SIZE - 1) // PAGE_SIZE for L in seq_lens)) if B else 1)
    swa_table = np.full((B, P_swa), poison_swa, dtype=np.int64)
    k = 0
    for r in range(B):
        for lp in swa_pages_per_req[r]:
            swa_table[r, lp] = perm[k]
            k += 1
    swa_pool = _alloc_pool(n_pages, kv)
    for r in range(B):
        pos = np.arange(tok_lo[r], seq_lens[r])
        slots = swa_table[r, pos // PAGE_SIZE] * PAGE_SIZE + pos % PAGE_SIZE
        _store_rows(swa_pool, kv, slots, tok_rows[r])

    # ---- extra (compressed) pages: every page of every request is backed ----
    extra_pool = extra_table = None
    poison_extra = -1
    if R:
        pages_per_req = [int((n + PAGE_SIZE - 1) // PAGE_SIZE) for n in n_ent]
        n_live = sum(pages_per_req)
        n_pages = n_live + max(1, int(round(decoy_frac * n_live))) + 1
        perm = rng.permutation(n_pages)
        poison_extra = int(perm[-1])
        P_extra = max(1, max(pages_per_req) if B else 1)
        extra_table = np.full((B, P_extra), poison_extra, dtype=np.int64)
        k = 0
        for r in range(B):
            for lp in range(pages_per_req[r]):
                extra_table[r, lp] = perm[k]
                k += 1
        extra_pool = _alloc_pool(n_pages, kv)
        for r in range(B):
            ids = cmp_ids[r]
            slots = extra_table[r, ids // PAGE_SIZE] * PAGE_SIZE + ids % PAGE_SIZE
            _store_rows(extra_pool, kv, slots, cmp_rows[r])

    logical = None
    if keep_logical:
        logical = [
            {
                "tok_lo": int(tok_lo[r]),
                "tok": tok_rows[r],
                "cmp_ids": cmp_ids[r] if R else np.zeros(0, np.int64),
                "cmp": cmp_rows[r] if R else None,
            }
            for r in range(B)
        ]

    return Case(
        name=name,
        H=H,
        W=W,
        R=R,
        kv=kv,
        scale=float(scale),
        seq_lens=seq_lens.astype(np.int32),
        qo_indptr=qo_indptr.astype(np.int32),
        q=q,
        sink=sink_arr,
        swa_pool=swa_pool,
        swa_page_table=swa_table.astype(np.int32),
        extra_pool=extra_pool,
        extra_page_table=None if extra_table is None else extra_table.astype(np.int32),
        c4_indices=None if c4 is None else c4.astype(np.int32),
        poison_swa_page=poison_swa,
        poison_extra_page=poison_extra,
        logical=logical,
        meta={"row_req": row_req, "row_pos": row_pos, "seed": seed,
              **({"c4_sets": np.stack(c4_sets).astype(np.int32)} if R == 4 and index_sets > 1 else {})},
    )


def tile_requests(case: Case, copies: int) -> Case:
    """A batch of ``copies`` x B requests made from a C4 case built with
    ``index_sets`` a multiple of ``copies`` (batch sweeps at full context
    length without backing every request's pool separately).

    Copy k of request r (request k*B + r) keeps r's sequence length, page
    tables, pools and Q rows and reads through the C4 lists of index set k;
    ``meta["c4_sets"]`` of the result holds group j of the original sets
    (sets j*copies .. j*copies + copies - 1, one per copy) as its set j.
    Every entry any original set names is backed, so every copy reads
    backed rows; copies of one request share physical pages, and their lists
    are independent draws."""
    if copies < 1:
        raise ValueError("copies >= 1")
    if copies == 1:
        return case
    sets = case.meta.get("c4_sets")
    if case.R != 4 or sets is None or sets.shape[0] < copies or sets.shape[0] % copies:
        raise ValueError("need a C4 case whose index_sets is a multiple of copies")
    T0 = case.T
    groups = sets.reshape(sets.shape[0] // copies, copies * T0, sets.shape[2])
    n_q = np.diff(case.qo_indptr.astype(np.int64))
    qo = np.zeros(copies * case.B + 1, dtype=np.int64)
    qo[1:] = np.cumsum(np.tile(n_q, copies))
    row_req = np.concatenate([case.meta["row_req"] + k * case.B for k in range(copies)])
    return Case(
        name=case.name,
        H=case.H,
        W=case.W,
        R=case.R,
        kv=case.kv,
        scale=case.scale,
        seq_lens=np.tile(case.seq_lens, copies),
        qo_indptr=qo.astype(np.int32),
        q=np.concatenate([case.q] * copies),
        sink=case.sink,
        swa_pool=case.swa_pool,
        swa_page_table=np.tile(case.swa_page_table, (copies, 1)),
        extra_pool=case.extra_pool,
        extra_page_table=np.tile(case.extra_page_table, (copies, 1)),
        c4_indices=np.ascontiguousarray(groups[0]),
        poison_swa_page=case.poison_swa_page,
        poison_extra_page=case.poison_extra_page,
        logical=None,
        meta={"row_req": row_req, "row_pos": np.tile(case.meta["row_pos"], copies), "seed": case.meta["seed"],
              "c4_sets": np.ascontiguousarray(groups), "copies": copies},
    )


# --------------------------------------------------------------------------
# The five workload shapes (decode and MTP target-verify)
# --------------------------------------------------------------------------
CONFIGS = {
    1: dict(
        name="swa_decode_b1_s200_h8",
        desc="SWA-only decode, 1 request, seq_len 200, 8 q heads / 1 KV head, window 128, one 256-token page",
    ),
    2: dict(
        name="c4_decode_b32_s4k-8k_h64",
        desc="C4 decode, batch 32, seq_len U[4096,8192], 64 q heads, window 128 + top-512 C4 entries",
    ),
    3: dict(
        name="c128_decode_b64_s128k_h64",
        desc="C128 decode, batch 64, seq_len 131072, 64 q heads, window 128 + all 1024 C128 entries",
    ),
    4: dict(
        name="c4_verify_b32x4_p32k-64k_h64",
        desc="C4 target-verify, batch 32 x 4 query rows, prefix U[32768,65536], per-row top-512 C4 entries",
    ),
    5: dict(
        name="c4_decode_fp8_b8_s1m_h64",
        desc="C4 decode, batch 8, seq_len 1048576 (262144 C4 candidates), top-512, FP8-packed KV",
    ),
    # Sparse prefill / extend: many query rows per request, each with its
    # own causal window and (C4) its own top-512 index list.
    6: dict(
        name="c4_prefill_b4x2048_p32k_h64",
        desc="C4 sparse prefill, 4 requests x 2048 new rows after a 32768-token prefix, per-row top-512 C4 entries",
    ),
    7: dict(
        name="c128_prefill_b4x2048_p32k_h64",
        desc="C128 prefill, 4 requests x 2048 new rows after a 32768-token prefix, every visible C128 entry",
    ),
}


def make_config(n: int, seed: Optional[int] = None, keep_logical: bool = False, batch: Optional[int] = None,
                index_sets: int = 1, rows: Optional[int] = None) -> Case:
    """Inputs for workload ``n`` (1..7); default seed ``1000 + n``.
    ``index_sets`` (C4 workloads): see make_case.  ``batch`` overrides the
    number of requests (for the prefill workloads, ``rows`` the rows per
    request)."""
    if seed is None:
        seed = 1000 + n
    name = CONFIGS[n]["name"]
    if n == 1:
        return make_case(seq_lens=[200], n_q=1, H=8, R=0, seed=seed, keep_logical=keep_logical, name=name)
    if n == 2:
        B = batch or 32
        sl = np.random.Generator(np.random.PCG64(seed + 7919)).integers(4096, 8192, size=B, endpoint=True)
        return make_case(seq_lens=sl, n_q=1, H=64, R=4, seed=seed, keep_logical=keep_logical,
                         index_sets=index_sets, name=name)
    if n == 3:
        B = batch or 64
        return make_case(seq_lens=[131072] * B, n_q=1, H=64, R=128, seed=seed, keep_logical=keep_logical, name=name)
    if n == 4:
        B = batch or 32
        pre = np.random.Generator(np.random.PCG64(seed + 7919)).integers(32768, 65536, size=B, endpoint=True)
        return make_case(seq_lens=pre + 4, n_q=4, H=64, R=4, seed=seed, keep_logical=keep_logical,
                         index_sets=index_sets, name=name)
    if n == 5:
        B = batch or 8
        return make_case(seq_lens=[1048576] * B, n_q=1, H=64, R=4, kv="fp8", seed=seed,
                         keep_logical=keep_logical, index_sets=index_sets, name=name)
    if n in (6, 7):
        B = batch or 4
        n_q = rows or 2048
        return make_case(seq_lens=[32768 + n_q] * B, n_q=n_q, H=64, R=4 if n == 6 else 128, seed=seed,
                         keep_logical=keep_logical, index_sets=index_sets if n == 6 else 1, name=name)
    raise KeyError(n)
