"""Sparse attention over the selected tokens on the GPU against the oracle:
bf16 outputs within half a bf16 ulp of the oracle's double-precision result
(plus the fp32 sums' share), the log-sum-exp, skipped entries, empty rows, page sizes and row
strides, and a full-size batch on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import ensure_built, log
import sparse_attention_indexer_page_amd as idx

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _run(case, scale, lse=True):
    R, k = case.R, case.k
    q = torch.from_numpy(case.q.view(np.int16)).cuda()
    data = torch.from_numpy(case.data).cuda()
    bt = torch.from_numpy(case.block_tables).cuda()
    ind = torch.from_numpy(case.indices).cuda()
    tl = torch.from_numpy(case.topk_lens).cuda()
    out = torch.full((R, 64, 512), -1, dtype=torch.int16, device="cuda")
    ls = torch.full((R, 64), float("nan"), dtype=torch.float32, device="cuda") if lse else None
    wsb = idx.idx_sparse_mla_workspace_size(R, k)
    ws = torch.empty(wsb // 4, dtype=torch.float32, device="cuda")
    kv = idx.make_mla_cache(case.page_size, case.num_pages, data, case.page_stride,
                            case.row_stride)
    idx.idx_sparse_mla_decode(q, kv, bt, case.block_tables.shape[1], case.lens.shape[0],
                              case.next_n, ind, tl, k, scale, out, ls, ws, wsb)
    torch.cuda.synchronize()
    o = out.cpu().view(torch.bfloat16).double().numpy()
    return o, (ls.cpu().numpy() if lse else None)


def _check(case, scale, got, got_lse, rows=None):
    ref, ref_lse = oracle.sparse_mla(case.q, case.data, case.page_stride, case.row_stride,
                                     case.page_size, case.num_pages, case.block_tables,
                                     case.next_n, case.indices, case.topk_lens, scale)
    rows = range(case.R) if rows is None else rows
    # the largest |latent value| in the cache (its bf16 rows; padding is 0)
    cmax = float(np.abs((case.data.view(np.uint16).astype(np.uint32) << 16).view(np.float32)).max())
    for r in rows:
        n = int(case.topk_lens[r])
        if n == 0 or np.all(case.indices[r, :n] < 0):
            assert np.all(got[r] == 0), "row %d: empty selection must give zeros" % r
            if got_lse is not None:
                assert np.all(np.isneginf(got_lse[r]))
            continue
        # The output's own bf16 rounding (half an ulp: 2^-8 relative), plus
        # what the fp32 sums over at most 2048 tokens and the probabilities
        # (carried to ~2^-16 by two bf16 parts) can add, against the largest
        # latent value |c|: 2048 * 2^-24 + 2^-16 < 2e-4.
        err = np.abs(got[r] - ref[r])
        bound = 2.0 ** -8 * np.abs(ref[r]) + 2e-4 * cmax
        assert np.all(err <= bound), "row %d: max err %.3e, worst err/bound %.3f" % (
            r, err.max(), (err / bound).max())
        if got_lse is not None:
            assert np.allclose(got_lse[r], ref_lse[r], rtol=1e-4, atol=1e-3), "row %d lse" % r


@pytest.mark.parametrize("P,next_n,row_stride,scale", [
    (64, 1, None, 0.0625), (64, 1, None, 3.0), (32, 2, 1040, 1.5), (256, 1, 1536, 0.5)])
def test_sparse_mla_matches_oracle(P, next_n, row_stride, scale):
    """Scales from nearly uniform weights to sharply peaked ones (score
    spread ~0.2 to ~8), so both the averaging and the softmax are tested."""
    log("sparse mla P %d next_n %d stride %s scale %g" % (P, next_n, row_stride, scale))
    case = synth.mla_case([300, 0, 129, 1000, 17], next_n=next_n, P=P, k=256,
                          row_stride=row_stride, seed=70 + P, holes=True)
    got, lse = _run(case, scale)
    _check(case, scale, got, lse)


def test_sparse_mla_one_chunk_per_row_and_odd_list_length():
    """300 rows (next_n 2) with lists of at most 100 entries: one chunk per
    row (no split), a list length that is not a multiple of the 32-token
    block, plus skipped entries."""
    log("sparse mla one chunk per row")
    rng = np.random.default_rng(73)
    lens = rng.integers(0, 400, size=150)
    lens[:3] = [0, 1, 101]
    case = synth.mla_case(lens, next_n=2, P=64, k=100, seed=74, holes=True)
    assert idx.idx_sparse_mla_workspace_size(case.R, case.k) == case.R * 64 * (512 + 2) * 4
    got, lse = _run(case, 0.8)
    _check(case, 0.8, got, lse)


def test_sparse_mla_full_size_sampled_rows():
    """64 rows, 2048 selected tokens each (the decode batch's top-k), page 64."""
    log("sparse mla full size")
    rng = np.random.default_rng(71)
    lens = rng.integers(2048, 8192 + 1, size=64)
    case = synth.mla_case(lens, next_n=1, P=64, k=2048, seed=72)
    got, lse = _run(case, 0.5)
    sub = synth.MlaCase(case.q[[0, 33, 63]], case.data, case.page_stride, case.row_stride,
                        case.page_size, case.num_pages, case.block_tables[[0, 33, 63]],
                        case.lens[[0, 33, 63]], 1, case.indices[[0, 33, 63]],
                        case.topk_lens[[0, 33, 63]], case.k)
    _check(sub, 0.5, got[[0, 33, 63]], lse[[0, 33, 63]])
