"""The opt-in device-side check of the decode contracts: planted violations
are counted and located, valid inputs and unused table entries pass, and a
captured graph clears the result on every replay."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import ensure_built, log
import sparse_attention_indexer_page_amd as idx

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _case():
    case = synth.decode_case([0, 100, 700, 64, 129, 1000, 5, 300], next_n=1, P=64, k=16,
                             W=1024, bt_width=16, seed=990, canary=False)
    return case


def _run(lens, bt, case, W):
    res = torch.full((4,), 12345, dtype=torch.int32, device="cuda")
    idx.idx_validate_decode(torch.from_numpy(lens).cuda(), len(lens), torch.from_numpy(bt).cuda(),
                            bt.shape[1], case.cache.page_size, case.cache.num_pages, W, res)
    torch.cuda.synchronize()
    return res.cpu().tolist()


def _expected(lens, bt, P, num_pages, W):
    """The contract, restated: bad lengths and out-of-pool entries of the
    pages a sequence's length makes visible (at most the table's width)."""
    cap = bt.shape[1] * P
    bad_len = [b for b, L in enumerate(lens) if L < 0 or (W > 0 and L > W) or L > cap]
    bad_ent = 0
    first_ent = -1
    for b, L in enumerate(lens):
        pages = min((int(L) + P - 1) // P, bt.shape[1]) if L > 0 else 0
        n = int(sum(1 for p in range(pages) if bt[b, p] < 0 or bt[b, p] >= num_pages))
        bad_ent += n
        if n and first_ent < 0:
            first_ent = b
    return [len(bad_len), bad_ent, bad_len[0] if bad_len else -1, first_ent]


def test_valid_decode_inputs_pass():
    log("validate: valid")
    case = _case()
    # unused table entries hold the 0x7fffffff sentinel: not visible, not counted
    assert (case.block_tables == synth.BT_SENTINEL).any()
    assert _run(case.lens.copy(), case.block_tables.copy(), case, case.W) == [0, 0, -1, -1]
    assert _run(case.lens.copy(), case.block_tables.copy(), case, 0) == [0, 0, -1, -1]


def test_planted_violations_are_counted_and_located():
    log("validate: planted")
    case = _case()
    lens, bt = case.lens.copy(), case.block_tables.copy()
    lens[2] = 1025                               # above W and the table
    bt[4, 1] = case.cache.num_pages              # visible page 1 of a 129-token sequence
    bt[5, 3] = -2                                # visible page of a 1000-token sequence
    lens[7] = bt.shape[1] * case.cache.page_size + 1   # beyond the table
    bt[1, 5] = -7                                # page 5 of a 100-token sequence: not visible
    P, npg = case.cache.page_size, case.cache.num_pages
    want = _expected(lens, bt, P, npg, case.W)
    # lengths past the table also expose that row's unused (sentinel) entries
    assert want[0] == 2 and want[2] == 2 and want[3] == 2 and want[1] > 2
    assert _run(lens, bt, case, case.W) == want
    # without the width bound the table bound still catches both
    want0 = _expected(lens, bt, P, npg, 0)
    assert want0 == want
    assert _run(lens, bt, case, 0) == want0
    # the width bound alone: 1000 tokens against a width of 800
    assert _expected(case.lens, case.block_tables, P, npg, 800) == [1, 0, 5, -1]
    assert _run(case.lens.copy(), case.block_tables.copy(), case, 800) == [1, 0, 5, -1]
    # the planted page ids alone, with valid lengths
    lens2 = case.lens.copy()
    want2 = _expected(lens2, bt, P, npg, case.W)
    assert want2 == [0, 2, -1, 4]
    assert _run(lens2, bt, case, case.W) == want2


def test_graph_replay_clears_the_result():
    log("validate: graph")
    case = _case()
    lens = torch.from_numpy(case.lens.copy()).cuda()
    bt = torch.from_numpy(case.block_tables.copy()).cuda()
    res = torch.empty(4, dtype=torch.int32, device="cuda")

    def check():
        idx.idx_validate_decode(lens, case.B, bt, bt.shape[1], case.cache.page_size,
                                case.cache.num_pages, case.W, res)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        check()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        check()
    for bad in (False, True, False):
        lens.copy_(torch.from_numpy(case.lens.copy()))
        if bad:
            lens[3] = case.W + 5
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = _expected(lens.cpu().numpy(), case.block_tables, case.cache.page_size,
                         case.cache.num_pages, case.W)
        assert want[0] == (1 if bad else 0)
        assert res.cpu().tolist() == want
