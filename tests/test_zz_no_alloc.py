"""idx_prefill_chunked_topk_noalloc, the prefill entry point for callers that
cannot allocate (its scratch is a fixed array in the library's device
memory), against idx_prefill_chunked_topk with caller-owned scratch on the
same inputs: identical selections on two calls in a row, the second smaller;
at the full chunked-prefill size, where the fixed 64 MiB logits scratch caps
the budget (five chunks instead of two) and the selection is still the same;
and replays of a captured graph of the call."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DeviceCase, ensure_built, log, run_prefill
import sparse_attention_indexer_page_amd as idx

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _noalloc(dc, budget, out=None, index_base=0):
    case = dc.case
    if out is None:
        out = torch.full((case.T, case.k), 12345, dtype=torch.int32, device="cuda")
    idx.idx_prefill_chunked_topk_noalloc(dc.query, dc.kv, dc.t["block_table"], dc.t["visible_end"],
                                         case.T, case.W, budget, case.k, index_base, out)
    return out


def test_noalloc_prefill_equals_the_caller_scratch_entry_two_calls():
    log("no-alloc prefill: two calls, the second smaller")
    first = synth.prefill_case(3000, 1000, P=64, k=256, W=1000, seed=777)
    second = synth.prefill_case(700, 300, P=32, k=64, W=300, dtype=synth.MXFP4, seed=778,
                                visible_end=np.minimum(np.arange(700) // 2 + 1, 300))
    for case, budget, base in ((first, 4 * 1000 * 3000, 0), (second, 4 * 300 * 100, 55)):
        dc = DeviceCase(case)
        _, want = run_prefill(dc, budget=budget, index_base=base)
        got = _noalloc(dc, budget, index_base=base)
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), want), "T=%d" % case.T


def test_noalloc_prefill_full_size_with_the_capped_budget():
    log("no-alloc prefill: chunked-prefill workload")
    case = synth.workload(4)
    assert 4 * case.W * case.T > idx.binding.IDX_NOALLOC_LOGITS_BYTES
    dc = DeviceCase(case)
    _, want = run_prefill(dc)
    got = _noalloc(dc, case.budget_bytes)
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), want)


def test_noalloc_prefill_in_a_captured_graph():
    log("no-alloc prefill: graph replays")
    case = synth.prefill_case(2500, 900, P=64, k=128, W=900, seed=779)
    dc = DeviceCase(case)
    _, want = run_prefill(dc, budget=4 * 900 * 600)
    out = torch.full((case.T, case.k), 12345, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _noalloc(dc, 4 * 900 * 600, out=out)  # first call on the device: the address lookup
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _noalloc(dc, 4 * 900 * 600, out=out)
    for i in range(3):
        out.fill_(777)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), want), "replay %d" % i
