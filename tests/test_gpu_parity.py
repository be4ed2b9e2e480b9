"""Parity of the HIP path with the CPU oracle on small cases that span several
tiles, blocks and pages plus ragged tails (every visible logit, every row)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import (DeviceCase, check_logits, check_topk_band, check_topk_exact, ensure_built,
                      log, oracle_decode_rows, oracle_prefill_rows, run_decode, run_prefill)
import sparse_attention_indexer_page_amd as idx

pytestmark = pytest.mark.gpu

# empty, one token, partial first page, page edges, several blocks, long tail
LENS = [0, 1, 17, 31, 32, 33, 64, 65, 100, 257, 1000, 2100]


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _check_decode(case, logits, out, cnt, label):
    rows = np.arange(case.R)
    ref, E = oracle_decode_rows(case, rows)
    lg = logits.numpy()
    for r in rows:
        what = "%s row %d (E=%d)" % (label, r, E[r])
        check_logits(lg[r], ref[r], E[r], what)
        assert np.all(np.isnan(lg[r, E[r]:])), what + ": wrote past the visible length"
        check_topk_band(out[r].numpy(), ref[r], E[r], case.k, what)
        assert cnt[r] == min(case.k, E[r])
    return ref, E


@pytest.mark.parametrize("P", [32, 64, 256])
@pytest.mark.parametrize("next_n", [1, 2, 3])
def test_decode_fp8(P, next_n):
    log("decode fp8 P=%d next_n=%d" % (P, next_n))
    case = synth.decode_case(LENS, next_n=next_n, P=P, k=64, W=2304, seed=100 + P + next_n)
    logits, out, cnt = run_decode(DeviceCase(case))
    _check_decode(case, logits, out, cnt, "fp8 P%d n%d" % (P, next_n))


@pytest.mark.parametrize("P", [32, 64, 256])
@pytest.mark.parametrize("next_n", [1, 2])
def test_decode_mxfp4(P, next_n):
    log("decode mxfp4 P=%d next_n=%d" % (P, next_n))
    case = synth.decode_case(LENS, next_n=next_n, P=P, k=64, W=2304, dtype=synth.MXFP4,
                             seed=200 + P + next_n)
    logits, out, cnt = run_decode(DeviceCase(case))
    _check_decode(case, logits, out, cnt, "mxfp4 P%d n%d" % (P, next_n))


@pytest.mark.parametrize("layout,row_stride", [("row_inline", 144), ("page_block", None),
                                               ("separate", 144)])
def test_decode_fp8_cache_layouts_give_identical_bits(layout, row_stride):
    log("layout %s stride %s" % (layout, row_stride))
    base = synth.decode_case(LENS, next_n=2, P=32, k=64, W=2304, seed=300)
    other = synth.decode_case(LENS, next_n=2, P=32, k=64, W=2304, seed=300, layout=layout,
                              row_stride=row_stride)
    la, oa, _ = run_decode(DeviceCase(base))
    lb, ob, cb = run_decode(DeviceCase(other))
    _check_decode(other, lb, ob, cb, "layout " + layout)
    assert torch.equal(torch.nan_to_num(la, nan=7.0), torch.nan_to_num(lb, nan=7.0))
    assert torch.equal(oa, ob)


@pytest.mark.parametrize("n_ctas", [1, 3, 64, 4096])
def test_schedule_split_does_not_change_results(n_ctas):
    log("n_ctas %d" % n_ctas)
    case = synth.decode_case(LENS, next_n=1, P=64, k=64, W=2304, seed=400)
    dc = DeviceCase(case)
    ref_l, ref_o, _ = run_decode(dc, n_ctas=512)
    l, o, _ = run_decode(dc, n_ctas=n_ctas)
    assert torch.equal(torch.nan_to_num(l, nan=7.0), torch.nan_to_num(ref_l, nan=7.0))
    assert torch.equal(o, ref_o)


@pytest.mark.parametrize("B,next_n,P,n_ctas", [(9, 1, 64, 512), (9, 2, 32, 3), (64, 1, 64, 2048),
                                               (130, 3, 256, 700), (1024, 1, 64, 1),
                                               (1024, 2, 32, 5000)])
def test_in_kernel_split_equals_the_schedule_buffer(B, next_n, P, n_ctas):
    """Without a schedule buffer each work group computes its own range; the
    logits and selections are bit-identical to the builder's split."""
    log("inline split B %d next_n %d P %d n_ctas %d" % (B, next_n, P, n_ctas))
    rng = np.random.default_rng(B + P)
    hi = 3000 if B <= 130 else 600
    lens = rng.integers(0, hi, size=B)
    lens[rng.integers(0, B, size=max(1, B // 8))] = 0
    lens[0] = hi - 1
    case = synth.decode_case(lens.tolist(), next_n=next_n, P=P, k=64, W=3000, seed=410 + B)
    dc = DeviceCase(case)
    ref_l, ref_o, ref_c = run_decode(dc, n_ctas=n_ctas)
    l, o, c = run_decode(dc, n_ctas=n_ctas, inline_split=True)
    assert torch.equal(torch.nan_to_num(l, nan=7.0), torch.nan_to_num(ref_l, nan=7.0))
    assert torch.equal(o, ref_o) and torch.equal(c, ref_c)
    if B <= 64:
        _check_decode(case, l, o, c, "inline split")


def test_physical_page_permutation_gives_identical_bits():
    case = synth.decode_case(LENS, next_n=1, P=32, k=64, W=2304, seed=500)
    la, oa, _ = run_decode(DeviceCase(case))
    c = case.cache
    perm = np.random.default_rng(1).permutation(c.num_pages)
    pages = c.data.reshape(c.num_pages, -1)
    spages = c.scale.reshape(c.num_pages, -1)
    nd, ns = np.empty_like(pages), np.empty_like(spages)
    nd[perm], ns[perm] = pages, spages
    c.data, c.scale = nd.reshape(-1), ns.reshape(-1)
    used = case.block_tables != synth.BT_SENTINEL
    case.block_tables[used] = perm[case.block_tables[used]]
    lb, ob, _ = run_decode(DeviceCase(case))
    assert torch.equal(torch.nan_to_num(la, nan=7.0), torch.nan_to_num(lb, nan=7.0))
    assert torch.equal(oa, ob)


def test_repeat_execution_is_bit_stable():
    case = synth.decode_case(LENS, next_n=2, P=64, k=64, W=2304, seed=600)
    dc = DeviceCase(case)
    first = run_decode(dc)
    for _ in range(3):
        again = run_decode(dc)
        assert torch.equal(torch.nan_to_num(first[0], nan=7.0), torch.nan_to_num(again[0], nan=7.0))
        assert torch.equal(first[1], again[1])


def test_bad_page_ids_read_zeros_instead_of_faulting():
    """A block-table entry outside the pool reads as an all-zero key block:
    those tokens score exactly 0 and every other logit is unchanged."""
    case = synth.decode_case([200, 130], next_n=1, P=32, k=16, W=256, seed=700, canary=False)
    good, _, _ = run_decode(DeviceCase(case))
    case.block_tables[0, 2] = case.cache.num_pages + 5  # tokens 64..95 of sequence 0
    case.block_tables[1, 1] = -3                          # tokens 32..63 of sequence 1
    bad, _, _ = run_decode(DeviceCase(case))
    assert torch.all(bad[0, 64:96] == 0) and torch.all(bad[1, 32:64] == 0)
    keep0 = torch.ones(200, dtype=torch.bool)
    keep0[64:96] = False
    assert torch.equal(bad[0, :200][keep0], good[0, :200][keep0])
    keep1 = torch.ones(130, dtype=torch.bool)
    keep1[32:64] = False
    assert torch.equal(bad[1, :130][keep1], good[1, :130][keep1])


@pytest.mark.parametrize("W,k", [(300, 1), (300, 64), (4096, 512), (5000, 2048), (65536, 2048)])
def test_topk_exact_on_oracle_logits(W, k):
    """idx_topk on the oracle's fp32 logits (uploaded) equals the oracle's
    top-k of the same values exactly, including planted ties and -0/+0."""
    log("topk exact W=%d k=%d" % (W, k))
    case = synth.decode_case([0, 1, min(W, 7), W // 3, W - 1, W], next_n=1, P=64, k=k, W=W,
                             seed=800 + k, H=64)
    rows = np.arange(case.R)
    ref, E = oracle_decode_rows(case, rows)
    f32 = ref.astype(np.float32)
    f32[~np.isfinite(f32)] = 0.0
    rng = np.random.default_rng(k)
    for r in rows:  # plant ties, including across -0/+0
        e = int(E[r])
        if e > 4:
            pick = rng.integers(0, e, size=max(e // 5, 2))
            f32[r, pick] = f32[r, pick[0]]
            f32[r, pick[:2]] = [0.0, -0.0]
    dev = torch.from_numpy(f32).cuda()
    lens = torch.from_numpy(case.lens).cuda()
    out = torch.empty((case.R, k), dtype=torch.int32, device="cuda")
    idx.idx_topk(dev, W, lens, case.B, 1, k, out)
    torch.cuda.synchronize()
    for r in rows:
        check_topk_exact(out[r].cpu().numpy(), f32[r], int(E[r]), k, "row %d" % r)


def _adversarial_rows(W, rng):
    """Score rows that exercise every path of the short-row selection: wide
    and narrow ranges, a crowded bin under far outliers (several refinement
    passes), heavy ties, and -0/+0."""
    rows = []
    rows.append(rng.standard_normal(W).astype(np.float32))
    wide = (rng.choice([-1.0, 1.0], W) * 10.0 ** rng.uniform(-30, 30, W)).astype(np.float32)
    rows.append(wide)
    crowd = (1.0 + 1e-6 * rng.standard_normal(W)).astype(np.float32)
    crowd[rng.integers(0, W, 5)] = [3e38, -3e38, 1e20, -1e-20, 7.0]
    rows.append(crowd)
    ties = rng.integers(-3, 4, W).astype(np.float32)
    ties[ties == 0] = -0.0
    ties[::7] = 0.0
    rows.append(ties)
    steps = np.repeat(rng.standard_normal(W // 100 + 1), 100)[:W].astype(np.float32)
    rows.append(steps)
    return rows


@pytest.mark.parametrize("E,k", [(65, 64), (1000, 1), (1000, 999), (1500, 700), (2049, 2048),
                                 (3000, 2048), (4096, 2048), (4096, 4095)])
def test_topk_short_rows_exact(E, k):
    """A few rows of width 4096 (fewer than 2048 rows: the one-work-group-per-
    row selection): exact against the oracle's top-k of the same fp32 values
    on adversarial rows."""
    W = 4096
    rng = np.random.default_rng(E * 7 + k)
    rows = _adversarial_rows(W, rng)
    vals = np.stack(rows)
    dev = torch.from_numpy(vals).cuda()
    lens = torch.full((len(rows),), E, dtype=torch.int32, device="cuda")
    out = torch.empty((len(rows), k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(len(rows), dtype=torch.int32, device="cuda")
    idx.idx_topk(dev, W, lens, len(rows), 1, k, out, cnt)
    torch.cuda.synchronize()
    assert torch.all(cnt.cpu() == min(k, E))
    for r in range(len(rows)):
        check_topk_exact(out[r].cpu().numpy(), vals[r], E, k, "E=%d k=%d row %d" % (E, k, r))


@pytest.mark.parametrize("k", [1, 64, 700, 999, 2048, 4095])
def test_topk_wave_kernel_adversarial_rows_exact(k):
    """2560 rows of width 4096 (>= 2048 rows: one wave per row): the five
    adversarial row families at lengths in each of the kernel's three key
    buckets (<= 1024, <= 2048, <= 4096 keys), plus rows no longer than k;
    every row exact against the oracle's top-k of the same fp32 values."""
    log("topk wave kernel k %d" % k)
    W, R = 4096, 2560
    rng = np.random.default_rng(4242 + k)
    buckets = [(k + 1, 1024), (max(k + 1, 1025), 2048), (max(k + 1, 2049), 4096)]
    buckets = [(lo, hi) for lo, hi in buckets if lo <= hi]
    vals = np.empty((R, W), dtype=np.float32)
    E = np.empty(R, dtype=np.int32)
    fams = None
    for r in range(R):
        if r % 5 == 0:
            fams = _adversarial_rows(W, rng)
        vals[r] = fams[r % 5]
        if r % 17 == 16:  # everything visible is selected
            E[r] = rng.integers(0, k + 1)
        else:
            lo, hi = buckets[(r // 5) % len(buckets)]
            E[r] = rng.integers(lo, hi + 1)
    dev = torch.from_numpy(vals).cuda()
    lens = torch.from_numpy(E).cuda()
    out = torch.empty((R, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(R, dtype=torch.int32, device="cuda")
    idx.idx_topk(dev, W, lens, R, 1, k, out, cnt)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.array_equal(cnt.cpu().numpy(), np.minimum(E, k))
    for r in range(R):
        check_topk_exact(o[r], vals[r], int(E[r]), k, "k=%d row %d (E=%d)" % (k, r, E[r]))


def _sampled_positions(E):
    """Row positions whose scores the wide-row selection samples for its
    threshold estimate: the first 16 of every 256."""
    p = np.arange(E)
    return p[(p % 256) < 16]


@pytest.mark.parametrize("k", [64, 700, 2048])
def test_topk_wide_rows_every_threshold_path_exact(k):
    """Rows wider than 4096 scores (one work group per row, keys estimated
    from a sample): families that take each branch of the estimate -- keys
    above it compacted and selected with every tie taken (normal scores) or
    only some (runs of equal scores), too many keys above it (heavy ties, a
    crowded bin under far outliers) and too few (the sampled positions hold
    the largest scores) -- at several lengths; every row exact against the
    oracle's top-k of the same fp32 values. Two more families place the
    estimate below +0 (every score negative: the slots past a row's end then
    pass it too and must be left out) and among runs of -0/+0 (most scores
    signed zeros, a few positive), and the lengths leave the last wave of each
    key bucket part-filled."""
    log("topk wide rows k %d" % k)
    W = 65536
    rng = np.random.default_rng(9000 + k)
    vals, E = [], []
    for e in (4097, 20000, 32768, 40000, 65536):
        fams = _adversarial_rows(W, rng)
        boosted = rng.standard_normal(W).astype(np.float32)
        boosted[_sampled_positions(e)] += 100.0
        fams.append(boosted)
        fams.append((-1.0 - np.abs(rng.standard_normal(W))).astype(np.float32))
        zeros = np.where(rng.random(W) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        pos = rng.random(W) < 0.03
        zeros[pos] = np.abs(rng.standard_normal(int(pos.sum()))).astype(np.float32) + 0.5
        neg = rng.random(W) < 0.3
        zeros[neg] = -np.abs(rng.standard_normal(int(neg.sum()))).astype(np.float32) - 0.5
        fams.append(zeros)
        for row in fams:
            vals.append(row)
            E.append(e)
    vals = np.stack(vals)
    E = np.array(E, dtype=np.int32)
    dev = torch.from_numpy(vals).cuda()
    lens = torch.from_numpy(E).cuda()
    out = torch.empty((len(E), k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(len(E), dtype=torch.int32, device="cuda")
    idx.idx_topk(dev, W, lens, len(E), 1, k, out, cnt)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.array_equal(cnt.cpu().numpy(), np.minimum(E, k))
    for r in range(len(E)):
        check_topk_exact(o[r], vals[r], int(E[r]), k, "k=%d row %d (E=%d)" % (k, r, E[r]))


def test_topk_all_equal_and_two_values():
    W, k = 3000, 100
    rows = np.zeros((3, W), dtype=np.float32)
    rows[1, ::2] = 1.0
    rows[2] = -0.0
    rows[2, 1::3] = 0.0
    dev = torch.from_numpy(rows).cuda()
    lens = torch.full((3,), W, dtype=torch.int32, device="cuda")
    out = torch.empty((3, k), dtype=torch.int32, device="cuda")
    idx.idx_topk(dev, W, lens, 3, 1, k, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.array_equal(o[0], np.arange(k))
    assert np.array_equal(o[1], np.arange(0, 2 * k, 2))
    assert np.array_equal(o[2], np.arange(k))


@pytest.mark.parametrize("P", [32, 64, 256])
@pytest.mark.parametrize("dtype", [synth.FP8, synth.MXFP4])
def test_prefill_small_matches_oracle_and_is_chunk_invariant(dtype, P):
    """Every row against the oracle, then budgets of 4, 43 and 301 uneven
    chunks (each chunk's schedule built by the one schedule launch) give the
    same selection; pages of 32 rows use the two-tile key blocks."""
    log("prefill small dtype %d P %d" % (dtype, P))
    T = 301
    ve = np.minimum(2 * (np.arange(T) + 1), 600)  # ragged, several key blocks
    case = synth.prefill_case(T, 600, visible_end=ve, P=P, k=32, W=600, dtype=dtype,
                              seed=900 + dtype + P)
    dc = DeviceCase(case)
    full_budget = 4 * case.W * case.T
    scratch, out = run_prefill(dc, budget=full_budget)
    rows = np.arange(case.T)
    ref, E = oracle_prefill_rows(case, rows)
    lg = scratch.numpy().reshape(case.T, case.W)
    for r in rows:
        # rows seeing at most k keys select them all: their scores are only
        # computed when a longer row shares their block of fifteen rows
        if E[r] > case.k:
            check_logits(lg[r], ref[r], E[r], "prefill row %d" % r)
        check_topk_band(out[r].numpy(), ref[r], E[r], case.k, "prefill row %d" % r)
    # the first row block (rows 0-14, at most 30 <= k keys each) is not
    # scored at all: its scratch rows keep the NaN fill
    assert np.all(np.isnan(lg[:15]))
    for budget in (4 * case.W * 100, 4 * case.W * 7, 4 * case.W, 1):
        _, o2 = run_prefill(dc, budget=budget)
        assert torch.equal(o2, out), "budget %d changed the selection" % budget
    # GLOBAL output: the same selection shifted by the sequence's first token
    # in the batch's key order (padding stays -1), in both top-k kernels
    for budget in (full_budget, 4 * case.W * 7):
        _, og = run_prefill(dc, budget=budget, index_base=1_000_003)
        want = torch.where(out >= 0, out + 1_000_003, out)
        assert torch.equal(og, want), "index_base at budget %d" % budget


def test_prefill_global_indices_in_the_one_wave_top_k():
    """2100 rows of width 300: the chunk's top-k runs one wave per row; the
    GLOBAL selection is the local one shifted by index_base."""
    log("prefill global indices, wave top-k")
    T = 2100
    ve = np.minimum(np.arange(T) // 7 + 1, 300)
    case = synth.prefill_case(T, 300, visible_end=ve, P=64, k=40, W=300, seed=950)
    dc = DeviceCase(case)
    _, out = run_prefill(dc, budget=4 * case.W * T)
    _, og = run_prefill(dc, budget=4 * case.W * T, index_base=77)
    assert torch.equal(og, torch.where(out >= 0, out + 77, out))
    assert int((out >= 0).sum(dim=1).min()) == 1  # row 0 sees one token


@pytest.mark.parametrize("next_n", [1, 3])
def test_fill_flag_sets_the_tail_to_minus_inf(next_n):
    """With IDX_QUERY_FILL_NEG_INF the columns [E_r, W) of every row read -inf
    and the visible columns are bit-identical to a run without the flag."""
    log("fill flag next_n %d" % next_n)
    case = synth.decode_case([0, 1, 5, 300, 1999], next_n=next_n, P=32, k=16, W=2003, seed=960)
    dc = DeviceCase(case)
    ref_l, ref_o, _ = run_decode(dc, n_ctas=64)
    dc.query = idx.make_query(case.dtype, dc.t["q"], dc.t["q_scale"], dc.t["w"],
                              flags=idx.IDX_QUERY_FILL_NEG_INF)
    l, o, _ = run_decode(dc, n_ctas=64, inline_split=True)
    lg, rl = l.numpy(), ref_l.numpy()
    for r in range(case.R):
        b, j = divmod(r, next_n)
        e = max(0, int(case.lens[b]) - (next_n - 1 - j))
        assert np.array_equal(lg[r, :e], rl[r, :e])
        assert np.all(np.isneginf(lg[r, e:])), "row %d tail" % r
    assert torch.equal(o, ref_o)
