"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks the oracle against what a library routine, exact rational
arithmetic, a closed-form special case or an invariant of the definition
fixes, so that a dropped term, a wrong sign or index, or a transposed operand
anywhere in the oracle fails at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _cache(case):
    c = case.cache
    return oracle.Cache(c.dtype, c.data, c.page_stride, c.row_stride, c.scale,
                        c.scale_page_stride, c.scale_row_stride, c.page_size, c.num_pages)


def _decode_all(case, W=None):
    W = W or case.W
    rows = np.arange(case.R)
    return oracle.decode_logits(case.dtype, case.q, case.q_scale, case.w, case.H, case.D,
                                _cache(case), case.block_tables, case.lens, case.next_n,
                                rows, W)


# ------------------------------------------------------------------ decoders

def test_fp8_decoder_matches_torch_for_all_256_codes():
    """OCP E4M3FN decoding against torch's float8_e4m3fn -> float32 cast."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.dec_fp8(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ref[~nan], got[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e2m1_decoder_matches_ocp_value_table():
    """The 16 E2M1 codes decode to the OCP MX value set, sign in bit 3."""
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = [oracle.dec_e2m1(c) for c in range(16)]
    assert got[:8] == table
    assert got[8:] == [-v for v in table]
    assert math.copysign(1.0, got[8]) == -1.0


def test_e8m0_decoder_anchor_doubling_and_nan():
    assert oracle.dec_e8m0(127) == 1.0
    for b in range(254):
        assert oracle.dec_e8m0(b + 1) == 2.0 * oracle.dec_e8m0(b)
    assert math.isnan(oracle.dec_e8m0(255))


def test_quantizers_round_trip_through_oracle_decoders():
    """Input quantizers (synth) and oracle decoders agree on what a code means:
    dequantized values stay within each format's rounding bound of the input."""
    rng = synth.rng_for(5)
    x = rng.standard_normal((64, 128), dtype=np.float32)
    codes, scale = synth.quantize_fp8_rows(x)
    dec = np.vectorize(oracle.dec_fp8)(codes) * scale[:, None].astype(np.float64)
    # E4M3: 3 mantissa bits -> relative error <= 2^-4 for normals; absolute
    # error <= half the subnormal step (2^-10 * scale) near zero.
    err = np.abs(dec - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[:, None])
    assert np.all(err <= bound * (1 + 1e-6))
    packed, sc = synth.quantize_mxfp4(x)
    lo = packed & 15
    hi = packed >> 4
    nib = np.empty((64, 128), dtype=np.uint8)
    nib[:, 0::2] = lo
    nib[:, 1::2] = hi
    vals = np.vectorize(oracle.dec_e2m1)(nib)
    s = np.vectorize(oracle.dec_e8m0)(sc)
    dq = vals * np.repeat(s, 32, axis=1)
    # block max sits in [4, 8) * 2^e; E2M1 spacing there is 2 * 2^e, so the
    # error is <= 2^e (half step) everywhere in the block, plus saturation at 6
    # for values in (6, 8) * 2^e (error < 2 * 2^e).
    step = np.repeat(s, 32, axis=1)
    assert np.all(np.abs(dq - x) <= 2.0 * step + 1e-12)
    assert np.all(np.sign(dq)[np.abs(dq) > 0] == np.sign(x)[np.abs(dq) > 0])


# ------------------------------------------------------- exact brute force

def _fp8_exact(code):
    v = torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item()
    return Fraction(v)


def _f32_exact(b4):
    return Fraction(float(np.frombuffer(bytes(b4), dtype=np.float32)[0]))


def _brute_force_decode_fp8(case, r):
    """Exact rational logits of decode row r: walks the block table by hand."""
    c = case.cache
    b, j = divmod(r, case.next_n)
    E = max(0, int(case.lens[b]) - (case.next_n - 1 - j))
    qs = Fraction(float(case.q_scale[r]))
    q = [[_fp8_exact(int(case.q[r, h, d])) * qs for d in range(case.D)]
         for h in range(case.H)]
    out = []
    for t in range(E):
        page = int(case.block_tables[b, t // c.page_size])
        slot = t % c.page_size
        base = page * c.page_stride + slot * c.row_stride
        if c.scale_offset >= 0:
            sb = c.scale_offset + page * c.scale_page_stride + slot * c.scale_row_stride
            ks = _f32_exact(c.data[sb:sb + 4])
        else:
            sb = page * c.scale_page_stride + slot * c.scale_row_stride
            ks = _f32_exact(c.scale[sb:sb + 4])
        k = [_fp8_exact(int(c.data[base + d])) * ks for d in range(case.D)]
        total = Fraction(0)
        for h in range(case.H):
            s = sum(qa * kb for qa, kb in zip(q[h], k))
            if s > 0:
                total += Fraction(float(case.w[r, h])) * s
        out.append(total)
    return out


@pytest.mark.parametrize("layout,row_stride", [("separate", None), ("row_inline", 144),
                                               ("page_block", None)])
def test_oracle_matches_exact_rational_brute_force_fp8(layout, row_stride):
    case = synth.decode_case([0, 5, 37], next_n=2, P=32, H=3, D=32, k=8, W=40,
                             layout=layout, row_stride=row_stride, seed=11)
    got, E = _decode_all(case)
    for r in range(case.R):
        exact = _brute_force_decode_fp8(case, r)
        assert E[r] == len(exact)
        for t, ex in enumerate(exact):
            ref = float(ex)
            assert abs(got[r, t] - ref) <= 1e-12 * max(abs(ref), 1e-30), (r, t)
        assert np.all(np.isneginf(got[r, len(exact):]))


def test_oracle_mxfp4_matches_exact_rational_brute_force():
    case = synth.decode_case([3, 33], next_n=1, P=32, H=2, D=64, k=4, dtype=synth.MXFP4,
                             seed=12)
    got, E = _decode_all(case)
    c = case.cache
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]

    def nib_val(n):
        v = Fraction(table[n & 7])
        return -v if n & 8 else v

    for r in range(case.R):
        q = []
        for h in range(case.H):
            row = []
            for d in range(case.D):
                byte = int(case.q[r, h, d // 2])
                n = byte & 15 if d % 2 == 0 else byte >> 4
                row.append(nib_val(n) * Fraction(2) ** (int(case.q_scale[r, h, d // 32]) - 127))
            q.append(row)
        for t in range(int(E[r])):
            page = int(case.block_tables[r, t // c.page_size])
            base = page * c.page_stride + (t % c.page_size) * c.row_stride
            sb = page * c.scale_page_stride + (t % c.page_size) * c.scale_row_stride
            k = []
            for d in range(case.D):
                byte = int(c.data[base + d // 2])
                n = byte & 15 if d % 2 == 0 else byte >> 4
                k.append(nib_val(n) * Fraction(2) ** (int(c.scale[sb + d // 32]) - 127))
            ex = Fraction(0)
            for h in range(case.H):
                s = sum(a * b for a, b in zip(q[h], k))
                if s > 0:
                    ex += Fraction(float(case.w[r, h])) * s
            assert abs(got[r, t] - float(ex)) <= 1e-12 * max(abs(float(ex)), 1e-30)


# -------------------------------------------- special cases and invariants

def _dense_keys_fp8(case, b):
    """Logical keys of sequence b, dequantized through torch's FP8 cast and
    gathered with numpy indexing (a path independent of the oracle's walk)."""
    c = case.cache
    P = c.page_size
    L = int(case.lens[b])
    pages = case.block_tables[b, :(L + P - 1) // P].astype(np.int64)
    rows = (pages[:, None] * P + np.arange(P)).reshape(-1)[:L]
    data = c.data.reshape(c.num_pages * P, c.row_stride)[rows, :case.D]
    kf = torch.from_numpy(np.ascontiguousarray(data)).view(torch.float8_e4m3fn).double().numpy()
    ks = c.scale.view(np.float32)[rows].astype(np.float64)
    return kf * ks[:, None]


def test_single_head_unit_weight_reduces_to_relu_matvec():
    """H=1, w=1: logits = max(0, K q) (numpy matmul on torch-decoded values)."""
    case = synth.decode_case([70, 1, 128], next_n=1, P=32, H=1, D=128, k=4, seed=21)
    case.w[:] = 1.0
    got, E = _decode_all(case)
    for b in range(case.B):
        kf = _dense_keys_fp8(case, b)
        qf = torch.from_numpy(case.q[b, 0].copy()).view(torch.float8_e4m3fn).double().numpy()
        qf = qf * float(case.q_scale[b])
        ref = np.maximum(kf @ qf, 0.0)
        assert np.allclose(got[b, :E[b]], ref, rtol=1e-13, atol=0)


def test_identical_heads_with_mean_weights_equal_single_head():
    """All heads equal and w = 1/H gives exactly the single-head relu(K q)
    (up to double rounding)."""
    case = synth.decode_case([90], next_n=1, P=32, H=8, D=128, k=4, seed=22)
    case.q[:, 1:] = case.q[:, :1]
    case.w[:] = 1.0 / 8.0
    got, E = _decode_all(case)
    kf = _dense_keys_fp8(case, 0)
    qf = torch.from_numpy(case.q[0, 0].copy()).view(torch.float8_e4m3fn).double().numpy()
    ref = np.maximum(kf @ (qf * float(case.q_scale[0])), 0.0)
    assert np.allclose(got[0, :E[0]], ref, rtol=1e-12, atol=0)


def test_multi_head_matches_dense_matmul_formulation():
    """Paged oracle vs a dense numpy formulation relu(Q K^T) w on gathered keys."""
    case = synth.decode_case([200, 64, 33], next_n=2, P=32, H=16, D=128, k=8, seed=23)
    got, E = _decode_all(case)
    for r in range(case.R):
        b = r // 2
        kf = _dense_keys_fp8(case, b)
        qf = torch.from_numpy(case.q[r].copy()).view(torch.float8_e4m3fn).double().numpy()
        qf = qf * float(case.q_scale[r])
        S = qf @ kf.T                                  # [H, L]
        ref = (np.maximum(S, 0.0) * case.w[r].astype(np.float64)[:, None]).sum(axis=0)
        e = int(E[r])
        assert e == max(0, int(case.lens[b]) - (1 - r % 2))
        scale = max(np.abs(ref[:e]).max() if e else 1.0, 1e-30)
        assert np.max(np.abs(got[r, :e] - ref[:e]), initial=0.0) <= 1e-12 * scale


def test_physical_page_permutation_is_invisible():
    case = synth.decode_case([100, 77], next_n=1, P=32, H=4, D=128, k=8, seed=24,
                             pool_pages=20)
    base, _ = _decode_all(case)
    c = case.cache
    perm = np.random.default_rng(3).permutation(c.num_pages)
    pages = c.data.reshape(c.num_pages, -1)
    spages = c.scale.reshape(c.num_pages, -1)
    new_data = np.empty_like(pages)
    new_scale = np.empty_like(spages)
    new_data[perm] = pages
    new_scale[perm] = spages
    c.data = new_data.reshape(-1)
    c.scale = new_scale.reshape(-1)
    bt = case.block_tables.copy()
    used = bt != synth.BT_SENTINEL
    bt[used] = perm[bt[used]]
    case.block_tables = bt
    moved, _ = _decode_all(case)
    assert np.array_equal(base, moved)


def test_canaries_and_sentinels_never_reach_visible_logits():
    """NaN canaries in tail slots/unreferenced pages and sentinels in unused
    block-table entries leave every visible logit finite and unchanged."""
    a = synth.decode_case([45, 3, 64], next_n=2, P=32, H=4, D=128, k=8, seed=25, canary=True)
    b = synth.decode_case([45, 3, 64], next_n=2, P=32, H=4, D=128, k=8, seed=25, canary=False)
    la, Ea = _decode_all(a)
    lb, Eb = _decode_all(b)
    assert np.array_equal(Ea, Eb)
    for r in range(a.R):
        assert np.all(np.isfinite(la[r, :Ea[r]]))
    assert np.array_equal(la, lb)


def test_mtp_rows_equal_single_row_calls_with_shorter_lengths():
    case = synth.decode_case([50, 1, 0], next_n=3, P=32, H=4, D=128, k=8, seed=26)
    got, E = _decode_all(case)
    for r in range(case.R):
        b, j = divmod(r, 3)
        one = synth.decode_case([50, 1, 0], next_n=3, P=32, H=4, D=128, k=8, seed=26)
        one.lens = np.maximum(case.lens - (3 - 1 - j), 0).astype(np.int32)
        one.next_n = 1
        one.q = case.q[j::3].copy()
        one.q_scale = case.q_scale[j::3].copy()
        one.w = case.w[j::3].copy()
        ref, Er = oracle.decode_logits(one.dtype, one.q, one.q_scale, one.w, one.H, one.D,
                                       _cache(one), one.block_tables, one.lens, 1, [b], case.W)
        assert Er[0] == E[r]
        assert np.array_equal(ref[0], got[r])


def test_key_scale_doubling_and_weight_negation_are_exact():
    case = synth.decode_case([60], next_n=1, P=32, H=4, D=128, k=8, seed=27, canary=False)
    base, E = _decode_all(case)
    case.cache.scale = (case.cache.scale.view(np.float32) * np.float32(2)).view(np.uint8)
    doubled, _ = _decode_all(case)
    assert np.array_equal(doubled[0, :E[0]], 2 * base[0, :E[0]])
    case.cache.scale = (case.cache.scale.view(np.float32) / np.float32(2)).view(np.uint8)
    case.w = -case.w
    neg, _ = _decode_all(case)
    assert np.array_equal(neg[0, :E[0]], -base[0, :E[0]])


def test_mxfp4_scale_byte_increment_doubles_logits():
    case = synth.decode_case([40], next_n=1, P=32, H=2, D=128, k=8, dtype=synth.MXFP4,
                             seed=28, canary=False)
    base, E = _decode_all(case)
    case.cache.scale = (case.cache.scale + 1).astype(np.uint8)
    got, _ = _decode_all(case)
    assert np.array_equal(got[0, :E[0]], 2 * base[0, :E[0]])


def test_empty_history_gives_no_logits_and_no_selection():
    case = synth.decode_case([0, 0], next_n=2, P=32, H=4, D=128, k=8, W=16, seed=29)
    got, E = _decode_all(case)
    assert np.all(E == 0) and np.all(np.isneginf(got))
    assert np.all(oracle.topk(got[0], 0, 8) == -1)


def test_prefill_rows_match_decode_rows_of_same_keys():
    """A prefill row with visible_end e scores exactly like a one-row decode of
    the same keys with length e."""
    pc = synth.prefill_case(40, 96, P=32, H=4, D=128, k=8, seed=30)
    rows = np.arange(pc.T)
    got, E = oracle.prefill_logits(pc.dtype, pc.q, pc.q_scale, pc.w, pc.H, pc.D,
                                   _cache(pc), pc.block_table, pc.visible_end, rows, pc.W)
    assert np.array_equal(E, np.minimum((rows + 1) // 4, 96))
    bt = pc.block_table[None, :]
    for r in (0, 3, 7, 39):
        ref, Er = oracle.decode_logits(pc.dtype, pc.q[r:r + 1], pc.q_scale[r:r + 1],
                                       pc.w[r:r + 1], pc.H, pc.D, _cache(pc), bt,
                                       np.array([pc.visible_end[r]]), 1, [0], pc.W)
        assert Er[0] == E[r]
        assert np.array_equal(ref[0], got[r])


# ------------------------------------------------------------------- top-k

def _lexsort_topk(v, E, k):
    idx = np.lexsort((np.arange(E), -v[:E].astype(np.float64)))
    out = np.full(k, -1, dtype=np.int32)
    n = min(k, E)
    out[:n] = idx[:n]
    return out


@pytest.mark.parametrize("E,k", [(1, 1), (5, 8), (100, 7), (1000, 64), (4096, 512)])
def test_topk_matches_numpy_lexsort(E, k):
    rng = np.random.default_rng(E * 31 + k)
    v = rng.standard_normal(E).astype(np.float32)
    v[rng.integers(0, E, size=E // 4)] = v[0]  # plant ties
    got = oracle.topk(v, E, k)
    assert np.array_equal(got, _lexsort_topk(v, E, k))
    sel = got[got >= 0]
    rest = np.setdiff1d(np.arange(E), sel)
    if len(rest) and len(sel):
        assert v[sel].min() >= v[rest].max()


def test_topk_ties_go_to_lower_index_and_signed_zeros_are_equal():
    v = np.array([0.0, -0.0, 1.0, 0.0, -0.0, 1.0, -1.0], dtype=np.float32)
    got = oracle.topk(v, 7, 4)
    assert list(got) == [2, 5, 0, 1]
    v2 = np.full(10, 3.5, dtype=np.float32)
    assert list(oracle.topk(v2, 10, 3)) == [0, 1, 2]


def test_topk_pads_with_minus_one_when_row_is_short():
    v = np.array([2.0, 1.0, 3.0], dtype=np.float32)
    assert list(oracle.topk(v, 3, 6)) == [2, 0, 1, -1, -1, -1]
    assert list(oracle.topk(v, 0, 2)) == [-1, -1]


def test_topk_rows_f32_matches_per_row():
    rng = np.random.default_rng(9)
    lg = rng.standard_normal((5, 300)).astype(np.float32)
    E = np.array([0, 1, 299, 300, 150])
    out = oracle.topk_rows_f32(lg, E, 16)
    for i in range(5):
        assert np.array_equal(out[i], _lexsort_topk(lg[i], E[i], 16))


# ------------------------------------------------------------ K-cache writer

def _e4m3_values():
    return np.array([oracle.dec_fp8(c) for c in range(0x7F)])  # 0..448, no NaN


def test_fp8_encoder_matches_torch_cast():
    """The oracle's E4M3 encoder (nearest by table search, ties to even) equals
    torch's float8_e4m3fn cast on representable values, midpoints (ties),
    near-midpoints, subnormals and random values, both signs."""
    v = _e4m3_values()
    mids = (v[1:] + v[:-1]) / 2
    rng = np.random.default_rng(5)
    ys = np.concatenate([v, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                         np.nextafter(mids.astype(np.float32), np.float32(1e9)),
                         rng.standard_normal(2000) * 50, rng.uniform(0, 2 ** -6, 500)])
    ys = ys[np.abs(ys) <= 448].astype(np.float32)
    ys = np.concatenate([ys, -ys])
    want = torch.from_numpy(ys).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.enc_fp8(float(y)) for y in ys], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_fp8_row_quantizer_bounds():
    """Per-row FP8: the largest magnitude maps to 448 exactly, every value is
    within half a code step of x/scale, and an all-zero row has scale 1."""
    rng = np.random.default_rng(6)
    for scale in (1e-3, 1.0, 37.0):
        x = (rng.standard_normal(128) * scale).astype(np.float32)
        codes, s = oracle.quant_fp8_row(x)
        vals = np.array([oracle.dec_fp8(int(c)) for c in codes])
        assert np.max(np.abs(vals)) == 448.0
        y = x.astype(np.float64) / s
        step = np.where(np.abs(y) < 2 ** -6, 2.0 ** -9,
                        2.0 ** (np.floor(np.log2(np.maximum(np.abs(y), 2 ** -6))) - 3))
        assert np.all(np.abs(vals - y) <= step / 2 + 1e-12)
    codes, s = oracle.quant_fp8_row(np.zeros(128, np.float32))
    assert s == 1.0 and not codes.any()


def test_mxfp4_encoder_is_nearest_with_even_ties():
    """Per 32-element block: the block maximum scales into [4, 8), every code is
    the nearest E2M1 magnitude of |x|*2^-e (distance checked against all eight),
    an exact tie takes the even code, and zero never carries a sign."""
    mags = np.array([oracle.dec_e2m1(c) for c in range(8)])
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(256) * 3).astype(np.float32)
    x[:8] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.0]   # ties after e = 0 scaling
    x[8] = 7.9
    packed, sc = oracle.quant_mxfp4_row(x)
    codes = np.empty(256, dtype=np.int64)
    codes[0::2], codes[1::2] = packed & 15, packed >> 4
    for b in range(8):
        e = int(sc[b]) - 127
        y = x[32 * b:32 * b + 32].astype(np.float64) * 2.0 ** -e
        if b > 0:
            assert 4 <= np.max(np.abs(y)) < 8
        for i in range(32):
            c = int(codes[32 * b + i])
            mag = c & 7
            d = np.abs(mags - min(abs(y[i]), 1e300))
            assert d[mag] == d.min()
            if np.sum(d == d.min()) > 1:
                assert mag % 2 == 0
            assert (c & 8) == (8 if (y[i] < 0 and mag > 0) else 0)
    # block 0 holds 7.9 -> e = 0: the ties above resolve to the even codes
    assert list(codes[:7] & 7) == [0, 2, 2, 4, 4, 6, 6]


def test_writer_encoders_agree_with_the_input_generator():
    """The oracle's encoders give the same bytes as the generator the scoring
    tests run on (an independent implementation: torch cast / thresholds)."""
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((20, 128)) * rng.uniform(1e-3, 50, (20, 1))).astype(np.float32)
    x[3] = 0.0
    x[4, 5] = -0.0
    codes, scales = synth.quantize_fp8_rows(x)
    packed, sc = synth.quantize_mxfp4(x)
    for r in range(20):
        c, s = oracle.quant_fp8_row(x[r])
        assert np.array_equal(c, codes[r]) and np.float32(s) == scales[r]
        p, e = oracle.quant_mxfp4_row(x[r])
        assert np.array_equal(p, packed[r]) and np.array_equal(e, sc[r])


def test_oracle_kv_write_scatters_and_skips():
    """Rows land at page*P + slot of their slot_mapping entry with their own
    quantized bytes; a negative slot or a page past the pool writes nothing."""
    P, pages = 32, 4
    for dtype, db in ((synth.FP8, 128), (synth.MXFP4, 64)):
        cache = synth._alloc_cache(dtype, pages, P, 128, None, "separate", True)
        data0, scale0 = cache.data.copy(), cache.scale.copy()
        rng = np.random.default_rng(9)
        k = rng.standard_normal((6, 128)).astype(np.float32)
        sm = np.array([5, -1, 3 * P + 31, pages * P, 0, 40])
        oracle.kv_write(dtype, k, sm, oracle.Cache(dtype, cache.data, cache.page_stride,
                                                   cache.row_stride, cache.scale,
                                                   cache.scale_page_stride,
                                                   cache.scale_row_stride, P, pages))
        touched = np.zeros(cache.data.shape, bool)
        for t, s in enumerate(sm):
            if s < 0 or s >= pages * P:
                continue
            want = oracle.quant_fp8_row(k[t])[0] if dtype == synth.FP8 else \
                oracle.quant_mxfp4_row(k[t])[0]
            off = (s // P) * cache.page_stride + (s % P) * cache.row_stride
            assert np.array_equal(cache.data[off:off + db], want)
            touched[off:off + db] = True
        assert np.array_equal(cache.data[~touched], data0[~touched])
        changed_scales = np.nonzero(cache.scale != scale0)[0] // 4
        assert set(changed_scales.tolist()) <= {5, 3 * P + 31, 0, 40}


# ------------------------------------------------------ query quantization

def _query_rows(R, seed, H=64, D=128):
    """Query rows whose heads differ in magnitude by up to 2^12, with exact
    zeros, a zero head and a zero row mixed in."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, H, D)).astype(np.float32)
    x *= np.exp2(rng.integers(-6, 7, size=(R, H, 1))).astype(np.float32)
    x[:, :, ::17] = 0.0
    if R > 1:
        x[1, 3] = 0.0
    if R > 2:
        x[2] = 0.0
    return x


def test_query_fp8_quantizer_matches_torch_cast_and_folds_the_scale():
    """FP8 query rows: one fp32 scale per row, amax/448 (numpy single
    precision; 1 for the zero row); codes equal torch's float8_e4m3fn cast of
    x/s; folded weights are (w*s)*c and unfolded ones w*c with s returned."""
    x = _query_rows(5, 41)
    w = np.random.default_rng(42).standard_normal((5, 64)).astype(np.float32)
    c = np.float32(0.125 * 0.0883883)
    q, qs, wf = oracle.quantize_query(oracle.FP8, x, w, c, fold=True)
    q2, qs2, wu = oracle.quantize_query(oracle.FP8, x, w, c, fold=False)
    assert qs is None and np.array_equal(q, q2)
    amax = np.abs(x.reshape(5, -1)).max(axis=1)
    s = np.where(amax > 0, amax / np.float32(448), np.float32(1)).astype(np.float32)
    assert s[2] == 1.0 and np.array_equal(qs2, s)
    want = torch.from_numpy(x / s[:, None, None]).to(torch.float8_e4m3fn)
    assert np.array_equal(q, want.view(torch.uint8).numpy())
    assert np.array_equal(wf, (w * s[:, None]) * c)
    assert np.array_equal(wu, w * c)


def test_query_mxfp4_quantizer_is_the_block_quantizer_per_head():
    """MXFP4 query rows: each head's 128 values carry four E8M0 bytes and
    their E2M1 codes exactly as the (separately pinned) block quantizer makes
    them; weights are w*c; dequantized values stay within half an E2M1 step
    of x (steps 0.5 / 1 / 2 times 2^e below 2 / 4 / 6), or at 6*2^e for
    |x| in [6, 8)*2^e (saturation; the block maximum is below 8*2^e)."""
    x = _query_rows(3, 43)
    w = np.random.default_rng(44).standard_normal((3, 64)).astype(np.float32)
    q, qs, wo = oracle.quantize_query(oracle.MXFP4, x, w, np.float32(2.0))
    assert q.shape == (3, 64, 64) and qs.shape == (3, 64, 4)
    for r in range(3):
        for h in range(64):
            p, sc = oracle.quant_mxfp4_row(x[r, h])
            assert np.array_equal(q[r, h], p) and np.array_equal(qs[r, h], sc)
    assert np.array_equal(wo, w * np.float32(2.0))
    nib = np.stack([q & 15, q >> 4], axis=-1).reshape(3, 64, 128)
    mag = np.array([oracle.dec_e2m1(int(n)) for n in range(16)])[nib]
    e = qs.astype(np.int64) - 127
    deq = mag * np.exp2(np.repeat(e, 32, axis=-1))
    y = np.abs(x) / np.exp2(np.repeat(e, 32, axis=-1))
    assert np.all(y < 8)
    ulp = np.exp2(np.repeat(e, 32, axis=-1))
    allowed = np.where(y < 2, 0.25, np.where(y < 4, 0.5, np.where(y <= 6, 1.0, y - 6))) * ulp
    assert np.all(np.abs(deq - x) <= allowed * (1 + 1e-6))
    assert np.all(np.sign(deq) * np.sign(x) >= 0)


def test_folded_and_unfolded_queries_score_alike_and_near_the_real_query():
    """Scoring the folded FP8 query (q_scale dropped, s in the weights) equals
    scoring the unfolded one up to rounding, because max(0, s*y) = s*max(0, y)
    for s > 0; both are close to the scores of the unquantized query against
    the same keys (E4M3 keeps 3 mantissa bits: each q element within 2^-4
    relative, so each head's dot product within 2^-4 of sum |q_i k_i|)."""
    case = synth.decode_case([150, 70], next_n=1, P=64, H=64, D=128, k=8, seed=45,
                             canary=False)
    x = _query_rows(2, 46)
    w = case.w.astype(np.float32)
    c = np.float32(0.5)
    qf, _, wf = oracle.quantize_query(oracle.FP8, x, w, c, fold=True)
    qu, su, wu = oracle.quantize_query(oracle.FP8, x, w, c, fold=False)
    case.q, case.q_scale, case.w = qf, None, wf
    folded, E = _decode_all(case)
    case.q, case.q_scale, case.w = qu, su, wu
    unfolded, _ = _decode_all(case)
    # the real query against the same dequantized keys, in float64; an E4M3
    # element is within 2^-4 relative when normal and within 2^-10 * s when
    # subnormal, and max(0, .) is 1-Lipschitz
    for r in range(2):
        n = E[r]
        assert n > 0
        keys = _dense_keys_fp8(case, r)
        scale = np.abs(unfolded[r, :n]).max()
        assert np.max(np.abs(folded[r, :n] - unfolded[r, :n])) <= 1e-6 * scale
        x64 = x[r].astype(np.float64)
        dots = x64 @ keys.T
        err = np.abs(x64) * 2.0 ** -4 + float(su[r]) * 2.0 ** -10
        real = (w[r, :, None].astype(np.float64) * c * np.maximum(dots, 0)).sum(axis=0)
        bound = (np.abs(w[r, :, None]) * c * (err @ np.abs(keys).T)).sum(axis=0)
        assert np.all(np.abs(unfolded[r, :n] - real) <= bound * (1 + 1e-9) + 1e-12)
        assert np.max(np.abs(unfolded[r, :n] - real)) <= 0.05 * np.abs(real).max()


# ------------------------------------------------------------ ragged decode

def test_varlen_windows_worked_example():
    """Sequences of lengths 10, 5, 0, 7, 2 owning 2, 1, 0, 4, 1 packed rows of a
    12-row buffer: each sequence's last row sees its whole length and each
    earlier draft row one key less (10: 9, 10; 5: 5; 7: 4, 5, 6, 7; 2: 2); the
    four rows nobody owns see nothing."""
    E = oracle.varlen_windows([10, 5, 0, 7, 2], [0, 2, 3, 3, 7, 8], 12)
    assert E.tolist() == [9, 10, 5, 4, 5, 6, 7, 2, 0, 0, 0, 0]


def test_varlen_with_rectangular_offsets_is_the_mtp_rule():
    """Offsets b*n give the rectangular step: the same windows and the same
    logits, bit for bit, as the next_n rule."""
    case = synth.decode_case([0, 1, 3, 64, 100], next_n=3, P=32, H=8, D=128, k=8, seed=47,
                             canary=False)
    off = (np.arange(case.B + 1) * 3).astype(np.int32)
    rect, E = _decode_all(case)
    assert np.array_equal(oracle.varlen_windows(case.lens, off, case.R), E)
    got, E2 = oracle.varlen_logits(case.dtype, case.q, case.q_scale, case.w, case.H, case.D,
                                   _cache(case), case.block_tables, case.lens, off, case.R,
                                   np.arange(case.R), case.W)
    assert np.array_equal(E2, E)
    assert np.array_equal(got, rect)


def test_varlen_rows_match_dense_formulation():
    """Packed ragged rows (0 to 4 per sequence) against a dense numpy
    relu(Q K^T) w over each owner's gathered keys; unowned rows see nothing."""
    case = synth.decode_case([50, 0, 130, 7, 64, 1], next_n=4, P=32, H=16, D=128, k=8, seed=48,
                             canary=False)
    off = synth.ragged_offsets(np.random.default_rng(49), case.B, 4)
    got, E = oracle.varlen_logits(case.dtype, case.q, case.q_scale, case.w, case.H, case.D,
                                  _cache(case), case.block_tables, case.lens, off, case.R,
                                  np.arange(case.R), case.W)
    owner = np.full(case.R, -1)
    for b in range(case.B):
        owner[off[b]:off[b + 1]] = b
    assert np.all(E[owner < 0] == 0) and np.all(np.isneginf(got[owner < 0]))
    for r in np.nonzero(owner >= 0)[0]:
        b = owner[r]
        n, j = off[b + 1] - off[b], r - off[b]
        e = int(E[r])
        assert e == max(0, int(case.lens[b]) - (n - 1 - j))
        kf = _dense_keys_fp8(case, b)[:e]
        qf = torch.from_numpy(case.q[r].copy()).view(torch.float8_e4m3fn).double().numpy()
        qf = qf * float(case.q_scale[r])
        ref = (np.maximum(qf @ kf.T, 0.0) * case.w[r].astype(np.float64)[:, None]).sum(axis=0)
        scale = max(np.abs(ref).max() if e else 1.0, 1e-30)
        assert np.max(np.abs(got[r, :e] - ref), initial=0.0) <= 1e-12 * scale
        assert np.all(np.isneginf(got[r, e:]))


# ------------------------------------------- sparse attention over top-k

def _mla(case, scale):
    return oracle.sparse_mla(case.q, case.data, case.page_stride, case.row_stride,
                             case.page_size, case.num_pages, case.block_tables, case.next_n,
                             case.indices, case.topk_lens, scale)


def _mla_rows(case, b, tokens):
    """Latent rows of sequence b's tokens, decoded by torch from the pool."""
    P = case.page_size
    pages = case.block_tables[b, np.asarray(tokens) // P].astype(np.int64)
    rows = pages * P + np.asarray(tokens) % P
    raw = case.data.reshape(-1, case.row_stride)[rows, :2 * case.D]
    bits = np.ascontiguousarray(raw).view(np.int16)
    return torch.from_numpy(bits).view(torch.bfloat16).double().numpy()


def _q64(case, r):
    return torch.from_numpy(case.q[r].view(np.int16)).view(torch.bfloat16).double().numpy()


def test_sparse_mla_single_token_returns_its_row_and_scale_zero_the_mean():
    """One selected token: the softmax weight is 1 and every head returns
    that latent row; scale 0: uniform weights, the mean of the rows."""
    case = synth.mla_case([40, 70], next_n=1, P=32, k=8, D=64, H=4, seed=61)
    case.topk_lens[0] = 1
    out, lse = _mla(case, 0.3)
    c = _mla_rows(case, 0, [case.indices[0, 0]])
    assert np.array_equal(out[0], np.repeat(c, 4, axis=0))
    out0, lse0 = _mla(case, 0.0)
    mean = _mla_rows(case, 1, case.indices[1, :8]).mean(axis=0)
    assert np.allclose(out0[1], mean[None, :], rtol=0, atol=1e-12)
    assert np.allclose(lse0[1], np.log(8.0))


def test_sparse_mla_matches_dense_softmax_and_ignores_list_order():
    """Against torch float64 softmax(scale q c^T) c on the gathered rows, and
    the same result for a permuted selection list; skipped (-1) entries and
    an empty row (zeros, lse -inf)."""
    case = synth.mla_case([300, 0, 129], next_n=2, P=64, k=64, D=128, H=8, seed=62,
                          holes=True)
    scale = 0.07
    out, lse = _mla(case, scale)
    for r in range(case.R):
        b = r // 2
        n = int(case.topk_lens[r])
        sel = case.indices[r, :n]
        sel = sel[sel >= 0]
        if len(sel) == 0:
            assert np.all(out[r] == 0) and np.all(np.isneginf(lse[r]))
            continue
        c = torch.from_numpy(_mla_rows(case, b, sel))
        qd = torch.from_numpy(_q64(case, r))
        s = scale * (qd @ c.T)
        ref = torch.softmax(s, dim=1) @ c
        assert np.allclose(out[r], ref.numpy(), rtol=0, atol=1e-10)
        assert np.allclose(lse[r], torch.logsumexp(s, dim=1).numpy(), atol=1e-10)
    perm = case.indices.copy()
    for r in range(case.R):
        n = int(case.topk_lens[r])
        perm[r, :n] = np.random.default_rng(r).permutation(perm[r, :n])
    case.indices = perm
    out2, _ = _mla(case, scale)
    assert np.allclose(out2, out, rtol=0, atol=1e-12)
