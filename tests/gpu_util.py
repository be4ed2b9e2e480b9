"""Helpers of the GPU tests: run the HIP library on a synthetic case through
the C ABI, run the oracle on the same case, and compare with the acceptance
rules (logits within 2e-3 of each row's max |logit|; top-k sets equal apart
from ties inside the tolerance band)."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle
import synth
import sparse_attention_indexer_page_amd as idx

LOGIT_RTOL = 2e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def ensure_built():
    """Builds libidx.so when its sources changed since the last build, then
    loads it."""
    from sparse_attention_indexer_page_amd import build
    build.ensure_built()
    idx.load()


def oracle_cache(case):
    c = case.cache
    return oracle.Cache(c.dtype, c.data, c.page_stride, c.row_stride, c.scale,
                        c.scale_page_stride, c.scale_row_stride, c.page_size, c.num_pages)


class DeviceCase:
    """A synthetic case resident on the GPU plus its ABI descriptors."""

    def __init__(self, case, device="cuda"):
        self.case = case
        self.t = synth.to_device(case, device)
        c = case.cache
        kscale = self.t["kscale"]
        if kscale is None:
            kscale = self.t["kdata"].data_ptr() + self.t["kscale_offset"]
        self.query = idx.make_query(case.dtype, self.t["q"], self.t["q_scale"], self.t["w"])
        self.kv = idx.make_kv_cache(case.dtype, c.page_size, c.num_pages, self.t["kdata"],
                                    c.page_stride, c.row_stride, kscale, c.scale_page_stride,
                                    c.scale_row_stride)


def run_decode(dc: DeviceCase, n_ctas=None, fill=float("nan"), k=None, stream=None,
               inline_split=False):
    """Schedule + logits + top-k of a decode case; returns (logits, idx, count)
    as CPU tensors. inline_split: no schedule buffer (each work group computes
    its own range)."""
    case = dc.case
    k = k or case.k
    R = case.R
    dev = dc.t["q"].device
    if n_ctas is None:
        n_ctas = idx.idx_recommended_ctas(R)
    cta = torch.empty(idx.idx_schedule_ints(n_ctas), dtype=torch.int32, device=dev)
    logits = torch.full((R, case.W), fill, dtype=torch.float32, device=dev)
    out = torch.empty((R, k), dtype=torch.int32, device=dev)
    cnt = torch.empty(R, dtype=torch.int32, device=dev)
    if inline_split:
        cta = None
    else:
        idx.idx_build_schedule(dc.t["lens"], case.B, case.next_n, case.cache.page_size, n_ctas,
                               cta, stream=stream)
    idx.idx_paged_mqa_logits(dc.query, dc.kv, dc.t["block_tables"], case.block_tables.shape[1],
                             dc.t["lens"], case.B, case.next_n, cta, n_ctas, logits, case.W,
                             stream=stream)
    idx.idx_topk(logits, case.W, dc.t["lens"], case.B, case.next_n, k, out, cnt, stream=stream)
    torch.cuda.synchronize()
    return logits.cpu(), out.cpu(), cnt.cpu()


def run_prefill(dc: DeviceCase, budget=None, k=None, index_base=0):
    """Chunked prefill; returns (last chunk's logits scratch, idx) on the CPU."""
    case = dc.case
    k = k or case.k
    budget = case.budget_bytes if budget is None else budget
    dev = dc.t["q"].device
    T, W = case.T, case.W
    sb = idx.idx_prefill_scratch_bytes(T, W, budget)
    si = idx.idx_prefill_schedule_ints(T, W, budget)
    scratch = torch.full((sb // 4,), float("nan"), dtype=torch.float32, device=dev)
    cta = torch.empty(si, dtype=torch.int32, device=dev)
    out = torch.empty((T, k), dtype=torch.int32, device=dev)
    idx.idx_prefill_chunked_topk(dc.query, dc.kv, dc.t["block_table"], dc.t["visible_end"], T, W,
                                 budget, k, index_base, scratch, sb, cta, si, out)
    torch.cuda.synchronize()
    return scratch.cpu(), out.cpu()


def oracle_decode_rows(case, rows, W=None):
    return oracle.decode_logits(case.dtype, case.q, case.q_scale, case.w, case.H, case.D,
                                oracle_cache(case), case.block_tables, case.lens, case.next_n,
                                np.asarray(rows), W or case.W)


def oracle_prefill_rows(case, rows, W=None):
    return oracle.prefill_logits(case.dtype, case.q, case.q_scale, case.w, case.H, case.D,
                                 oracle_cache(case), case.block_table, case.visible_end,
                                 np.asarray(rows), W or case.W)


def check_logits(got_row, ref_row, E, what=""):
    """|got - ref| <= 2e-3 * max|ref| over t < E; nothing non-finite."""
    if E == 0:
        return 0.0
    g = np.asarray(got_row[:E], dtype=np.float64)
    r = np.asarray(ref_row[:E], dtype=np.float64)
    assert np.all(np.isfinite(g)), "%s: non-finite logits in the visible range" % what
    scale = max(np.abs(r).max(), np.finfo(np.float32).tiny)
    err = np.abs(g - r).max() / scale
    assert err <= LOGIT_RTOL, "%s: max error %.3e of row max" % (what, err)
    return err


def check_topk_band(got_idx, ref_row, E, k, what=""):
    """Top-k of the HIP path vs the oracle's exact top-k of its double logits:
    same size, distinct, in range, ascending; every element of the symmetric
    difference has an oracle logit within 2*tol of the oracle's k-th value."""
    got = np.asarray(got_idx)
    n = min(k, E)
    assert np.all(got[n:] == -1), "%s: padding is not -1" % what
    sel = got[:n]
    assert np.all((sel >= 0) & (sel < E)), "%s: index out of range" % what
    assert np.all(np.diff(sel) > 0), "%s: indices not strictly ascending" % what
    if E <= k:
        assert np.array_equal(sel, np.arange(E)), "%s: short row must select all" % what
        return 0
    ref = np.asarray(ref_row[:E], dtype=np.float64)
    ref_sel = oracle.topk(ref, E, k)
    theta = ref[ref_sel[k - 1]]
    tol = LOGIT_RTOL * max(np.abs(ref).max(), np.finfo(np.float32).tiny)
    diff = np.setxor1d(sel, ref_sel)
    if len(diff):
        far = np.abs(ref[diff] - theta) > 2 * tol
        assert not far.any(), "%s: %d selections differ outside the tie band" % (what, far.sum())
    return len(diff)


def check_topk_exact(got_idx, logits_f32_row, E, k, what=""):
    """idx_topk on the oracle's own fp32 logits equals the oracle's top-k of
    those same values, bit for bit (as an ascending set)."""
    ref = oracle.topk(np.ascontiguousarray(logits_f32_row[:max(E, 1)], dtype=np.float32), E, k)
    n = min(k, E)
    want = np.concatenate([np.sort(ref[:n]), np.full(k - n, -1, dtype=np.int32)])
    assert np.array_equal(np.asarray(got_idx), want), "%s: exact-input top-k differs" % what
