"""Brute-force dense attention over unpaged logical rows (tiny inputs only).

A second formulation of DSV4 decode/verify attention, used to pin the C
oracle: no page tables, no slot lists, no gather.  Each request's token rows
and compressed rows are laid out densely by logical position, every key gets
a boolean visibility mask (window ``p-W < x <= p``; C128 ``c < (p+1)//128``;
C4 membership in the row's index list) and one dense softmax runs over
``[tokens | compressed | sink]`` with numpy in fp64.  Storage decoding uses
torch's own bf16 and float8_e4m3fn conversions.
"""
from __future__ import annotations

import numpy as np
import torch


def decode_rows(rows) -> np.ndarray:
    """Storage rows -> float64 [n, 512] via torch's dtype conversions."""
    if isinstance(rows, tuple):
        codes, scales, rope = rows
        nope = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        nope = nope * scales.astype(np.float64)[:, None]
        rp = torch.from_numpy(np.ascontiguousarray(rope).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
        return np.concatenate([nope, rp], axis=1)
    return torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def dense_request(case, r: int):
    """Dense logical arrays of request r: tokens [L,512] and compressed [n,512] (NaN where absent)."""
    lg = case.logical[r]
    L = int(case.seq_lens[r])
    tok = np.full((L, 512), np.nan)
    rows = decode_rows(lg["tok"])
    tok[lg["tok_lo"]:L] = rows
    n_ent = L // case.R if case.R else 0
    cmp = np.full((n_ent, 512), np.nan)
    if case.R and len(lg["cmp_ids"]):
        cmp[lg["cmp_ids"]] = decode_rows(lg["cmp"])
    return tok, cmp


def attention(case, window=None):
    """(out [T,H,512], lse [T,H]) by dense masked softmax.  ``window`` overrides W."""
    W = case.W if window is None else window
    T, H = case.T, case.H
    out = np.zeros((T, H, 512))
    lse = np.zeros((T, H))
    q_all = bf16_bits_to_f64(case.q.reshape(T * H, 512)).reshape(T, H, 512)
    sink = None if case.sink is None else case.sink.astype(np.float64)
    dense = {}
    for t in range(T):
        r = int(np.searchsorted(case.qo_indptr, t, side="right") - 1)
        n_q = int(case.qo_indptr[r + 1] - case.qo_indptr[r])
        p = int(case.seq_lens[r]) - n_q + (t - int(case.qo_indptr[r]))
        if r not in dense:
            dense[r] = dense_request(case, r)
        tok, cmp = dense[r]
        x = np.arange(tok.shape[0])
        mtok = (x > p - W) & (x <= p)
        c = np.arange(cmp.shape[0])
        if case.R == 128:
            mcmp = c < (p + 1) // 128
        elif case.R == 4:
            mcmp = np.isin(c, case.c4_indices[t][case.c4_indices[t] >= 0])
        else:
            mcmp = np.zeros(0, bool)
        keys = np.concatenate([tok, cmp], axis=0)
        mask = np.concatenate([mtok, mcmp])
        keys = np.where(mask[:, None], keys, 0.0)
        q = q_all[t]                                  # [H, 512]
        s = case.scale * (keys @ q.T)                 # [N, H]
        s = np.where(mask[:, None], s, -np.inf)
        if sink is not None:
            s = np.concatenate([s, sink[None, :]], axis=0)
        m = s.max(axis=0)
        e = np.exp(s - m[None, :])
        z = e.sum(axis=0)
        lse[t] = m + np.log(z)
        out[t] = (e[: keys.shape[0]] / z[None, :]).T @ keys
    return out, lse
