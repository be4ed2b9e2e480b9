"""The decode step (schedule + scores + top-k) captured once in a HIP graph:
replays equal eager runs, also after the lengths and block tables were
rewritten in place (ATOM PR #1709, commits on the ragged-window refresh: a
replay must never read the previous step's metadata)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import (DeviceCase, check_logits, check_topk_band, ensure_built, log,
                      oracle_decode_rows, run_decode)
import sparse_attention_indexer_page_amd as idx

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _capture(dc, n_ctas):
    case = dc.case
    R, W, k = case.R, case.W, case.k
    cta = torch.empty(idx.idx_schedule_ints(n_ctas), dtype=torch.int32, device="cuda")
    logits = torch.full((R, W), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.empty((R, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(R, dtype=torch.int32, device="cuda")

    def step():
        idx.idx_build_schedule(dc.t["lens"], case.B, case.next_n, case.cache.page_size, n_ctas, cta)
        idx.idx_paged_mqa_logits(dc.query, dc.kv, dc.t["block_tables"], case.block_tables.shape[1],
                                 dc.t["lens"], case.B, case.next_n, cta, n_ctas, logits, W)
        idx.idx_topk(logits, W, dc.t["lens"], case.B, case.next_n, k, out, cnt)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    return g, logits, out, cnt


@pytest.mark.parametrize("next_n,P", [(1, 64), (2, 32)])
def test_graph_replay_matches_eager_after_in_place_metadata_update(next_n, P):
    log("graph next_n=%d P=%d" % (next_n, P))
    lens = [0, 1, 40, 100, 700, 1500, 2048, 33]
    case = synth.decode_case(lens, next_n=next_n, P=P, k=128, W=2048, seed=1200 + P)
    dc = DeviceCase(case)
    n_ctas = 256
    g, logits, out, cnt = _capture(dc, n_ctas)
    eager_l, eager_o, eager_c = run_decode(dc, n_ctas=n_ctas)
    for rep in range(3):
        logits.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.nan_to_num(logits.cpu(), nan=7.0),
                           torch.nan_to_num(eager_l, nan=7.0)), "replay %d" % rep
        assert torch.equal(out.cpu(), eager_o) and torch.equal(cnt.cpu(), eager_c)

    # New step: shorter/longer lengths (within each sequence's pages) and
    # pages moved to new physical ids; rewrite in place, then replay.
    rng = np.random.default_rng(5)
    new_lens = np.array([3, 0, 40, 64, 1999, 1500, 17, 33], dtype=np.int32)
    c = case.cache
    perm = rng.permutation(c.num_pages)
    pages = c.data.reshape(c.num_pages, -1)
    spages = c.scale.reshape(c.num_pages, -1)
    nd, ns = np.empty_like(pages), np.empty_like(spages)
    nd[perm], ns[perm] = pages, spages
    c.data, c.scale = nd.reshape(-1), ns.reshape(-1)
    used = case.block_tables != synth.BT_SENTINEL
    case.block_tables[used] = perm[case.block_tables[used]]
    case.lens = np.minimum(new_lens, case.lens)
    dc.t["kdata"].copy_(torch.from_numpy(c.data))
    dc.t["kscale"].copy_(torch.from_numpy(c.scale))
    dc.t["block_tables"].copy_(torch.from_numpy(case.block_tables))
    dc.t["lens"].copy_(torch.from_numpy(case.lens))
    torch.cuda.synchronize()
    logits.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    new_l, new_o, new_c = run_decode(dc, n_ctas=n_ctas)
    assert torch.equal(torch.nan_to_num(logits.cpu(), nan=7.0), torch.nan_to_num(new_l, nan=7.0))
    assert torch.equal(out.cpu(), new_o) and torch.equal(cnt.cpu(), new_c)
    rows = np.arange(case.R)
    ref, E = oracle_decode_rows(case, rows)
    for r in rows:
        check_logits(logits[r].cpu().numpy(), ref[r], E[r], "graph row %d" % r)
        check_topk_band(out[r].cpu().numpy(), ref[r], E[r], case.k, "graph row %d" % r)
