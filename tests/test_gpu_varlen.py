"""Ragged decode on the GPU: packed draft rows per sequence (0 to max_q of
them) with per-row windows built on the device. Windows equal the oracle's
exactly; logits of every owned row are within the logit tolerance of the
oracle, unowned rows and columns past each window are never written; the
top-k over the windows matches the oracle's selection; rectangular offsets
reproduce the rectangular entry bit for bit; a captured graph replays a new
step's offsets correctly (ATOM PR #1709, commits on the ragged varlen
windows)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (DeviceCase, check_logits, check_topk_band, ensure_built, log,
                      oracle_cache, run_decode)
import sparse_attention_indexer_page_amd as idx

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _step(dc, off_dev, max_q, n_ctas, logits, ve, out, cnt, inline_split=False):
    case = dc.case
    cta = None
    if not inline_split:
        cta = torch.empty(idx.idx_schedule_ints(n_ctas), dtype=torch.int32, device="cuda")
        idx.idx_build_schedule(dc.t["lens"], case.B, max_q, case.cache.page_size, n_ctas, cta)
    idx.idx_paged_mqa_logits_varlen(dc.query, dc.kv, dc.t["block_tables"],
                                    case.block_tables.shape[1], dc.t["lens"], off_dev, case.B,
                                    max_q, cta, n_ctas, logits, case.W)
    idx.idx_varlen_windows(dc.t["lens"], off_dev, case.B, max_q, ve)
    idx.idx_topk(logits, case.W, ve, case.B * max_q, 1, case.k, out, cnt)


def _buffers(case, max_q):
    R = case.B * max_q
    logits = torch.full((R, case.W), float("nan"), dtype=torch.float32, device="cuda")
    ve = torch.full((R,), -5, dtype=torch.int32, device="cuda")
    out = torch.empty((R, case.k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(R, dtype=torch.int32, device="cuda")
    return logits, ve, out, cnt


def _check(case, off, max_q, logits, ve, out, cnt):
    R = case.B * max_q
    E_ref = oracle.varlen_windows(case.lens, off, R)
    assert np.array_equal(ve.cpu().numpy(), E_ref), "windows differ from the oracle"
    ref, E = oracle.varlen_logits(case.dtype, case.q, case.q_scale, case.w, case.H, case.D,
                                  oracle_cache(case), case.block_tables, case.lens, off, R,
                                  np.arange(R), case.W)
    lg = logits.cpu().numpy()
    o, c = out.cpu().numpy(), cnt.cpu().numpy()
    owned = np.zeros(R, dtype=bool)
    owned[:off[-1]] = True
    for r in range(R):
        e = int(E[r])
        if not owned[r]:
            assert np.all(np.isnan(lg[r])), "unowned row %d was written" % r
        else:
            assert np.all(np.isnan(lg[r, e:])), "row %d written past its window" % r
            check_logits(lg[r], ref[r], e, "row %d" % r)
        assert c[r] == min(case.k, e)
        check_topk_band(o[r], ref[r], e, case.k, "row %d" % r)


@pytest.mark.parametrize("dtype,P,max_q,inline_split", [
    (synth.FP8, 64, 4, False), (synth.FP8, 32, 3, True), (synth.MXFP4, 256, 2, False),
    (synth.MXFP4, 64, 3, True), (synth.FP8, 256, 1, False)])
def test_varlen_matches_oracle(dtype, P, max_q, inline_split):
    log("varlen dtype %d P %d max_q %d inline %d" % (dtype, P, max_q, inline_split))
    rng = np.random.default_rng(300 + P + max_q)
    B = 24
    lens = rng.integers(0, 2500, size=B).astype(np.int32)
    lens[:5] = [0, 1, 2, 3, 4096]
    rng.shuffle(lens)
    case = synth.decode_case(lens.tolist(), next_n=max_q, P=P, dtype=dtype, k=200, W=4096,
                             seed=301 + P)
    off = synth.ragged_offsets(rng, B, max_q)
    dc = DeviceCase(case)
    bufs = _buffers(case, max_q)
    _step(dc, torch.from_numpy(off).cuda(), max_q, 300, *bufs, inline_split=inline_split)
    torch.cuda.synchronize()
    _check(case, off, max_q, *bufs)


@pytest.mark.parametrize("max_q,P", [(2, 32), (4, 64)])
def test_varlen_rectangular_offsets_equal_the_rectangular_entry(max_q, P):
    log("varlen rectangular max_q %d P %d" % (max_q, P))
    case = synth.decode_case([0, 5, 300, 1024, 77, 2000], next_n=max_q, P=P, k=64, W=2048,
                             seed=310 + P)
    dc = DeviceCase(case)
    rect_l, rect_o, rect_c = run_decode(dc, n_ctas=128)
    off = (np.arange(case.B + 1) * max_q).astype(np.int32)
    logits, ve, out, cnt = _buffers(case, max_q)
    _step(dc, torch.from_numpy(off).cuda(), max_q, 128, logits, ve, out, cnt)
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(logits.cpu(), nan=7.0), torch.nan_to_num(rect_l, nan=7.0))
    assert torch.equal(out.cpu(), rect_o) and torch.equal(cnt.cpu(), rect_c)


def test_varlen_graph_replays_new_offsets():
    """One captured graph (schedule, scores, windows, top-k) replayed over
    three steps whose draft counts and lengths differ, offsets and lengths
    rewritten in place between replays; every replay matches the oracle."""
    log("varlen graph")
    max_q, B = 3, 16
    rng = np.random.default_rng(320)
    lens0 = rng.integers(100, 1800, size=B).astype(np.int32)
    case = synth.decode_case(lens0.tolist(), next_n=max_q, P=64, k=128, W=2048, seed=321,
                             canary=False)
    dc = DeviceCase(case)
    off_dev = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    off_dev.copy_(torch.from_numpy((np.arange(B + 1) * max_q).astype(np.int32)))
    logits, ve, out, cnt = _buffers(case, max_q)
    n_ctas = 200
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(dc, off_dev, max_q, n_ctas, logits, ve, out, cnt)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    cta = torch.empty(idx.idx_schedule_ints(n_ctas), dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        idx.idx_build_schedule(dc.t["lens"], case.B, max_q, case.cache.page_size, n_ctas, cta)
        idx.idx_paged_mqa_logits_varlen(dc.query, dc.kv, dc.t["block_tables"],
                                        case.block_tables.shape[1], dc.t["lens"], off_dev, B,
                                        max_q, cta, n_ctas, logits, case.W)
        idx.idx_varlen_windows(dc.t["lens"], off_dev, B, max_q, ve)
        idx.idx_topk(logits, case.W, ve, B * max_q, 1, case.k, out, cnt)
    for step in range(3):
        off = synth.ragged_offsets(rng, B, max_q)
        # each step commits some tokens: lengths only grow within the pages held
        case.lens = np.minimum(lens0 + step * 7, (lens0 + 63) // 64 * 64).astype(np.int32)
        off_dev.copy_(torch.from_numpy(off))
        dc.t["lens"].copy_(torch.from_numpy(case.lens))
        logits.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log("varlen graph step %d: %d rows" % (step, int(off[-1])))
        _check(case, off, max_q, logits, ve, out, cnt)


def test_varlen_fill_flag_defines_every_row():
    """With IDX_QUERY_FILL_NEG_INF every row of the B*max_q buffer is defined:
    owned rows read -inf past their window, unowned rows are all -inf."""
    log("varlen fill flag")
    max_q = 3
    case = synth.decode_case([40, 0, 700, 65, 3], next_n=max_q, P=64, k=32, W=1000, seed=330)
    off = np.array([0, 2, 2, 5, 6, 7], dtype=np.int32)
    dc = DeviceCase(case)
    dc.query = idx.make_query(case.dtype, dc.t["q"], dc.t["q_scale"], dc.t["w"],
                              flags=idx.IDX_QUERY_FILL_NEG_INF)
    logits, ve, out, cnt = _buffers(case, max_q)
    _step(dc, torch.from_numpy(off).cuda(), max_q, 50, logits, ve, out, cnt)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    E = oracle.varlen_windows(case.lens, off, case.B * max_q)
    assert not np.isnan(lg).any(), "a logit was left unwritten"
    for r in range(case.B * max_q):
        assert np.all(np.isneginf(lg[r, E[r]:])), "row %d" % r
        assert np.all(np.isfinite(lg[r, :E[r]]))
