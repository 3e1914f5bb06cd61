"""Helpers for GPU tests: move a synthetic case to the GPU, run the HIP path,
and compare with the oracle at the stated tolerances.

Tolerances (bf16 inputs, fp32 accumulation, bf16 output rounded to nearest
even):  out within atol 2e-2 + rtol 2e-2 of the fp64 oracle, lse within 1e-3
absolute.  As a sharper diagnostic the per-(row, head) relative L2 error of
``out`` must stay below 1.5e-2: bf16 rounding of the output (2^-9) and of the
probabilities fed to the PV product (2^-9 per term, averaging out) give about
3e-3, so 1.5e-2 leaves a 5x margin.  Neither bound can see one dropped or
extra key among hundreds; the bit-exact slot lists and the spike tests do.
"""
from __future__ import annotations

import numpy as np
import torch

ATOL = 2e-2
RTOL = 2e-2
LSE_ATOL = 1e-3
REL_L2 = 1.5e-2


def to_gpu(case, device="cuda"):
    dev = torch.device(device)

    def t(a, dtype=None):
        if a is None:
            return None
        x = torch.from_numpy(np.ascontiguousarray(a))
        if dtype is not None:
            x = x.view(dtype)
        return x.to(dev)

    bf = torch.bfloat16
    g = {
        "q": t(case.q.view(np.int16), bf),
        "swa_pool": t(case.swa_pool.view(np.int16), bf) if case.kv == "bf16" else t(case.swa_pool),
        "swa_page_table": t(case.swa_page_table),
        "extra_pool": None,
        "extra_page_table": t(case.extra_page_table),
        "c4_indices": t(case.c4_indices),
        "seq_lens": t(case.seq_lens),
        "qo_indptr": t(case.qo_indptr),
        "sink": t(case.sink),
    }
    if case.extra_pool is not None:
        g["extra_pool"] = t(case.extra_pool.view(np.int16), bf) if case.kv == "bf16" else t(case.extra_pool)
    return g


def run_forward(case, g=None, **kw):
    from hybrid_sparse_mqa_amd import dsv4_attn_forward

    if g is None:
        g = to_gpu(case)
    out, lse = dsv4_attn_forward(
        g["q"], g["swa_pool"], g["swa_page_table"], g["extra_pool"], g["extra_page_table"], g["c4_indices"],
        g["seq_lens"], g["qo_indptr"], g["sink"], case.R, case.W, case.scale, **kw)
    torch.cuda.synchronize()
    return out, lse


def run_gather(case, g=None):
    from hybrid_sparse_mqa_amd import dsv4_attn_gather_slots

    if g is None:
        g = to_gpu(case)
    slots, counts = dsv4_attn_gather_slots(g["swa_page_table"], g["extra_page_table"], g["c4_indices"],
                                           g["seq_lens"], g["qo_indptr"], case.T, case.R, case.W)
    torch.cuda.synchronize()
    return slots.cpu().numpy(), counts.cpu().numpy()


def compare(out_gpu, lse_gpu, out_ref, lse_ref, rows=None, what=""):
    """Assert GPU results (torch, full) match oracle results (numpy, for `rows`)."""
    o = out_gpu.float().cpu().numpy().astype(np.float64)
    l_ = lse_gpu.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        o = o[rows]
        l_ = l_[rows]
    if o.size == 0:
        return 0.0, 0.0, 0.0
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - out_ref)
    bound = ATOL + RTOL * np.abs(out_ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} outputs off, max err {err.max():.3g}"
    le = np.abs(l_ - lse_ref)
    assert le.max() <= LSE_ATOL, f"{what}: lse off by {le.max():.3g}"
    num = np.sqrt(((o - out_ref) ** 2).sum(-1))
    den = np.sqrt((out_ref ** 2).sum(-1)) + 1e-30
    rel = num / den
    assert rel.max() <= REL_L2, f"{what}: relative L2 error {rel.max():.3g}"
    return float(err.max()), float(le.max()), float(rel.max())


def expected_keys(orc, case, t, compressed_first):
    """Row t's key list in a split kernel's order, from the oracle's canonical
    gather: entries ("swa" | "ext", physical slot), or None for an unused C4
    entry (the kernels keep its place, read the zero row and mask it out).
    compressed_first: the 32- and 64-head kernels' order (compressed entries,
    then the window); otherwise the window first."""
    swa, ext = orc.gather(case, t)
    swa_l = [("swa", int(s)) for s in swa]
    if case.R == 4:
        it = iter(ext)
        ext_l = [None if int(c) < 0 else ("ext", int(next(it))) for c in case.c4_indices[t]]
        assert next(it, None) is None
    else:
        ext_l = [("ext", int(s)) for s in ext]
    return ext_l + swa_l if compressed_first else swa_l + ext_l


def spike_slot(case, pool_name, slot, t, head=0, mult=8.0):
    """Overwrite physical slot `slot` of a pool with mult * q[t, head] (in the
    pool's storage format): that key dominates head `head` of row t if and
    only if the row reads it."""
    from synth import store_float_rows

    qv = torch.from_numpy(case.q[t, head].view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    store_float_rows(getattr(case, pool_name), case.kv, [slot], (mult * qv)[None, :])
