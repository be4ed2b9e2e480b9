"""Parity at the full sizes of the five measured workloads, in the launch
configuration the benchmark uses (recommended work-group count), checked on
sampled rows the oracle computes one by one, plus whole-output properties."""
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


def _check_sampled(case, logits, out, rows, label):
    ref, E = oracle_decode_rows(case, rows)
    lg = logits.numpy()
    for i, r in enumerate(rows):
        what = "%s row %d (E=%d)" % (label, r, E[i])
        check_logits(lg[r], ref[i], E[i], what)
        check_topk_band(out[r].numpy(), ref[i], E[i], case.k, what)
    return ref, E


def _exact_topk_on_oracle_logits(case, rows, ref, E):
    """idx_topk on the oracle's fp32 logits of the sampled rows, same W and k."""
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
    ref, E = _check_sampled(case, logits, out, [0], "w1")
    _exact_topk_on_oracle_logits(case, [0], ref, E)


def _bench_ctas(case):
    """The scoring launch configuration bench.py times for this workload."""
    n = idx.idx_recommended_decode_ctas(case.R, case.dtype, case.cache.page_size, case.next_n)
    assert n > 0
    return n


def test_recommended_decode_work_groups():
    """4 per CU for FP8 keys in 64-token blocks with one row per sequence,
    8 per CU otherwise, at least the row count; 0 for unsupported values."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert idx.idx_recommended_decode_ctas(64, synth.FP8, 64, 1) == 4 * cus
    assert idx.idx_recommended_decode_ctas(64, synth.FP8, 256, 1) == 4 * cus
    assert idx.idx_recommended_decode_ctas(64, synth.FP8, 32, 1) == 8 * cus
    assert idx.idx_recommended_decode_ctas(64, synth.FP8, 64, 2) == 8 * cus
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
    rng = np.random.default_rng(2)
    rows = sorted(set([0, case.R - 1] + list(rng.choice(case.R, 6, replace=False))))
    ref, E = _check_sampled(case, logits, out, rows, "w2")
    _exact_topk_on_oracle_logits(case, rows, ref, E)
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


def test_workload3_mtp_decode_page32_padded_rows():
    log("workload 3")
    case = synth.workload(3)
    logits, out, cnt = run_decode(DeviceCase(case), n_ctas=_bench_ctas(case),
                                  inline_split=True)
    _whole_output_properties(case, out, cnt, _decode_rows_E(case))
    rng = np.random.default_rng(3)
    forced = list(range(12))  # both MTP rows of the six edge-length sequences
    rows = sorted(set(forced + list(rng.choice(np.arange(12, case.R), 6, replace=False))))
    ref, E = _check_sampled(case, logits, out, rows, "w3")
    _exact_topk_on_oracle_logits(case, rows, ref, E)


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
    rows = [0, 2, 3, 4, 8191, 8192, 8195, 12000, 15624, 15625, 15626, 16000, 16383]
    ref, E = oracle_prefill_rows(case, rows)
    for i, r in enumerate(rows):
        check_topk_band(o[r], ref[i], E[i], k, "w4 row %d" % r)
    # logits of the second chunk are still in the scratch buffer
    lg = scratch.numpy()[: (T - c1) * W].reshape(T - c1, W)
    for i, r in enumerate(rows):
        if r >= c1:
            check_logits(lg[r - c1], ref[i], E[i], "w4 logits row %d" % r)
    # one chunk (the whole [T, W] buffer) gives identical indices
    scratch1, out1 = run_prefill(dc, budget=4 * W * T)
    assert torch.equal(out1, out)
    lg1 = scratch1.numpy().reshape(T, W)
    for i, r in enumerate(rows):
        check_logits(lg1[r], ref[i], E[i], "w4 one-chunk logits row %d" % r)


def test_workload5_mxfp4_decode():
    log("workload 5")
    case = synth.workload(5)
    logits, out, cnt = run_decode(DeviceCase(case), n_ctas=_bench_ctas(case),
                                  inline_split=True)
    _whole_output_properties(case, out, cnt, _decode_rows_E(case))
    rng = np.random.default_rng(5)
    rows = sorted(set([int(np.argmax(case.lens))] + list(rng.choice(case.R, 5, replace=False))))
    ref, E = _check_sampled(case, logits, out, rows, "w5")
    _exact_topk_on_oracle_logits(case, rows, ref, E)
