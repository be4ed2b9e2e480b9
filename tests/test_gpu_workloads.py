"""Parity at the full sizes of the five measured workloads, in the launch
configuration the benchmark uses (recommended work-group count): every row's
logits and top-k against the oracle, the top-k exactly on the oracle's own
fp32 logits, plus whole-output properties."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from gpu_util import (DeviceCase, check_logits, check_topk_band, check_topk_exact, ensure_built,
                      log, oracle_decode_rows, oracle_prefill_rows, run_decode, run_prefill)
import sparse_attention_indexer_page_amd as idx

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _whole_output_properties(case, out, cnt, E_all):
    """Every row: min(k, E) distinct ascending indices in [0, E), then -1."""
    o = out.numpy()
    c = cnt.numpy()
    for r in range(case.R):
        e = int(E_all[r])
        n = min(case.k, e)
        assert c[r] == n
        row = o[r]
        assert np.all(row[n:] == -1), "row %d padding" % r
        sel = row[:n]
        assert np.all((sel >= 0) & (sel < e)), "row %d range" % r
        assert np.all(np.diff(sel) > 0), "row %d order" % r


def _decode_rows_E(case):
    E = []
    for b in range(case.B):
        for j in range(case.next_n):
            E.append(max(0, int(case.lens[b]) - (case.next_n - 1 - j)))
    return np.array(E)


def _check_all_rows(case, logits, out, label, batch=32):
    """Every decode row: logits within tolerance and the top-k inside the tie
    band of the oracle's double logits, then idx_topk on the oracle's fp32
    logits bit-exact. The oracle runs a batch of rows at a time."""
    lg = logits.numpy()
    for r0 in range(0, case.R, batch):
        rows = np.arange(r0, min(r0 + batch, case.R))
        ref, E = oracle_decode_rows(case, rows)
        for i, r in enumerate(rows):
            what = "%s row %d (E=%d)" % (label, r, E[i])
            check_logits(lg[r], ref[i], E[i], what)
            check_topk_band(out[r].numpy(), ref[i], E[i], case.k, what)
        _exact_topk_on_oracle_logits(case, rows, ref, E)
    log("%s: all %d rows checked" % (label, case.R))


def _exact_topk_on_oracle_logits(case, rows, ref, E):
    """idx_topk on the oracle's fp32 logits of these rows, same W and k."""
    f32 = ref.astype(np.float32)
    f32[~np.isfinite(f32)] = 0.0
    dev = torch.from_numpy(f32).cuda()
    lens = torch.from_numpy(np.asarray(E, dtype=np.int32)).cuda()
    out = torch.empty((len(rows), case.k), dtype=torch.int32, device="cuda")
    idx.idx_topk(dev, case.W, lens, len(rows), 1, case.k, out)
    torch.cuda.synchronize()
    for i, r in enumerate(rows):
        check_topk_exact(out[i].cpu().numpy(), f32[i], int(E[i]), case.k, "exact row %d" % r)


def test_workload1_single_sequence_decode():
    log("workload 1")
    case = synth.workload(1)
    # the launch configuration bench.py times: no schedule buffer (B <= 1024)
    logits, out, cnt = run_decode(DeviceCase(case), inline_split=True)
    _whole_output_properties(case, out, cnt, _decode_rows_E(case))
    _check_all_rows(case, logits, out, "w1")


def _bench_ctas(case):
    """The scoring launch configuration bench.py times for this workload."""
    n = idx.idx_recommended_decode_ctas(case.R, case.dtype, case.cache.page_size, case.next_n)
    assert n > 0
    return n


def test_recommended_decode_work_groups():
    """4 per CU for FP8 keys in 64-token blocks, 8 per CU for smaller blocks
    where eight work groups' LDS fits a CU (up to three rows per sequence),
    else 4; at least the row count; 0 for unsupported values."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert idx.idx_recommended_decode_ctas(64, synth.FP8, 64, 1) == 4 * cus
    assert idx.idx_recommended_decode_ctas(64, synth.FP8, 256, 1) == 4 * cus
    assert idx.idx_recommended_decode_ctas(64, synth.FP8, 32, 1) == 8 * cus
    assert idx.idx_recommended_decode_ctas(64, synth.FP8, 64, 2) == 4 * cus  # 35 KB of LDS each
    assert idx.idx_recommended_decode_ctas(64, synth.FP8, 32, 3) == 8 * cus  # 20 KB: eight fit
    assert idx.idx_recommended_decode_ctas(64, synth.FP8, 32, 4) == 4 * cus  # 21 KB: seven would
    assert idx.idx_recommended_decode_ctas(64, synth.MXFP4, 256, 1) == 8 * cus
    assert idx.idx_recommended_decode_ctas(100000, synth.FP8, 64, 1) == 100000
    assert idx.idx_recommended_decode_ctas(64, 7, 64, 1) == 0
    assert idx.idx_recommended_decode_ctas(64, synth.FP8, 48, 1) == 0


def test_workload2_batched_decode_graph_replay():
    log("workload 2")
    case = synth.workload(2)
    dc = DeviceCase(case)
    n_ctas = _bench_ctas(case)
    logits, out, cnt = run_decode(dc, n_ctas=n_ctas, inline_split=True)
    _whole_output_properties(case, out, cnt, _decode_rows_E(case))
    _check_all_rows(case, logits, out, "w2")
    # the same step captured once and replayed gives the same bits, with the
    # schedule buffer as well as without it
    cta = torch.empty(idx.idx_schedule_ints(n_ctas), dtype=torch.int32, device="cuda")
    lg = torch.full_like(logits.cuda(), float("nan"))
    og = torch.empty_like(out.cuda())

    def step():
        idx.idx_build_schedule(dc.t["lens"], case.B, 1, case.cache.page_size, n_ctas, cta)
        idx.idx_paged_mqa_logits(dc.query, dc.kv, dc.t["block_tables"], case.block_tables.shape[1],
                                 dc.t["lens"], case.B, 1, cta, n_ctas, lg, case.W)
        idx.idx_topk(lg, case.W, dc.t["lens"], case.B, 1, case.k, og)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    assert torch.equal(og.cpu(), out)
    assert torch.equal(torch.nan_to_num(lg.cpu(), nan=7.0), torch.nan_to_num(logits, nan=7.0))

    # Metadata refresh at full size: the lengths and block tables are
    # rewritten in place (a second seed: every sequence takes another
    # sequence's pages and a new length no longer than theirs, so every
    # visible key is a written one), then the captured graph is replayed and
    # every row is checked against the oracle on the new metadata.
    rng = np.random.default_rng(20002)
    perm = rng.permutation(case.B)
    new_bt = np.ascontiguousarray(case.block_tables[perm])
    new_lens = np.array([rng.integers(1, int(case.lens[p]) + 1) for p in perm], dtype=np.int32)
    dc.t["lens"].copy_(torch.from_numpy(new_lens))
    dc.t["block_tables"].copy_(torch.from_numpy(new_bt))
    lg.fill_(float("nan"))
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    case2 = dataclasses.replace(case, lens=new_lens, block_tables=new_bt)
    cnt2 = torch.tensor([min(case.k, int(e)) for e in new_lens], dtype=torch.int32)
    _whole_output_properties(case2, og.cpu(), cnt2, _decode_rows_E(case2))
    _check_all_rows(case2, lg.cpu(), og.cpu(), "w2 refreshed")


def test_workload3_mtp_decode_page32_padded_rows():
    log("workload 3")
    case = synth.workload(3)
    logits, out, cnt = run_decode(DeviceCase(case), n_ctas=_bench_ctas(case),
                                  inline_split=True)
    _whole_output_properties(case, out, cnt, _decode_rows_E(case))
    _check_all_rows(case, logits, out, "w3")


def test_workload4_chunked_prefill():
    log("workload 4")
    case = synth.workload(4)
    dc = DeviceCase(case)
    assert idx.idx_prefill_rows_per_chunk(case.W, case.budget_bytes) == 15625
    T, W, k = case.T, case.W, case.k
    # two chunks (at most 15625 rows each), spread evenly: [0, 8192), [8192, 16384)
    c1 = idx.idx_prefill_scratch_bytes(T, W, case.budget_bytes) // (4 * W)
    assert c1 == 8192
    scratch, out = run_prefill(dc)
    E_all = case.visible_end.astype(np.int64)
    o = out.numpy()
    for r in range(T):  # whole output: short rows select everything
        e = int(E_all[r])
        n = min(k, e)
        assert np.all(o[r, n:] == -1)
        if e <= k:
            assert np.array_equal(o[r, :n], np.arange(n))
        else:
            assert np.all(np.diff(o[r, :n]) > 0) and o[r, 0] >= 0 and o[r, n - 1] < e
    # logits of the second chunk are still in the scratch buffer
    lg = scratch.numpy()[: (T - c1) * W].reshape(T - c1, W).copy()
    del scratch
    # one chunk (the whole [T, W] buffer) gives identical indices
    scratch1, out1 = run_prefill(dc, budget=4 * W * T)
    assert torch.equal(out1, out)
    lg1 = scratch1.numpy().reshape(T, W)
    # every row against the oracle, 1024 rows per oracle call: the top-k in
    # the tie band, and for the rows seeing more than k keys (the others
    # select every visible key and are not scored) the one-chunk logits and
    # the second chunk's logits
    for r0 in range(0, T, 1024):
        rows = np.arange(r0, min(r0 + 1024, T))
        ref, E = oracle_prefill_rows(case, rows)
        for i, r in enumerate(rows):
            check_topk_band(o[r], ref[i], E[i], k, "w4 row %d" % r)
            if E[i] > k:  # rows seeing at most k keys select them all, unscored
                check_logits(lg1[r], ref[i], E[i], "w4 one-chunk logits row %d" % r)
                if r >= c1:
                    check_logits(lg[r - c1], ref[i], E[i], "w4 logits row %d" % r)
    log("w4: all %d rows checked" % T)


def test_workload5_mxfp4_decode():
    log("workload 5")
    case = synth.workload(5)
    logits, out, cnt = run_decode(DeviceCase(case), n_ctas=_bench_ctas(case),
                                  inline_split=True)
    _whole_output_properties(case, out, cnt, _decode_rows_E(case))
    _check_all_rows(case, logits, out, "w5")
