"""Seeded synthetic inputs for the paged sparse-attention indexer.

This module serves both sides of every comparison (the CPU oracle and the HIP
library) and holds none of the indexer's arithmetic: no scoring, no ReLU or
head sum, no selection. It only

  * draws Gaussian queries, keys and per-head weights from a seeded PCG64
    generator,
  * quantizes them into the storage formats the cache uses (FP8 E4M3FN with a
    per-row fp32 scale, through torch's CPU cast; MXFP4 = E2M1 nibbles with one
    E8M0 scale per 32 elements, through the quantizer below),
  * lays the keys out in a shuffled page pool addressed by block tables, with
    NaN canaries in every byte no visible token owns.

The shapes, value distributions and length mixes follow the five workloads the
library is measured on (single-sequence decode, 64-sequence batched decode,
128-sequence MTP decode on 32-row pages, 16k-row chunked prefill, 128-sequence
MXFP4 decode); see ``workload``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

FP8 = 1
MXFP4 = 2

BT_SENTINEL = 0x7FFFFFFF  # unused block-table entries
FP8_CANARY = 0x7F         # E4M3FN NaN
E2M1_CANARY = 0x77        # two max-magnitude nibbles (E2M1 has no NaN)
E8M0_CANARY = 0xFF        # E8M0 NaN
F32_NAN_BYTES = np.array([0x7FC00000], dtype=np.uint32).view(np.uint8)


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


# ----------------------------------------------------------------- quantizers

def quantize_fp8_rows(x: np.ndarray):
    """Per-row FP8 E4M3FN: scale = amax/448 over everything but axis 0.

    Returns (codes uint8 with x's shape, scale float32 [N])."""
    n = x.shape[0]
    flat = np.ascontiguousarray(x, dtype=np.float32).reshape(n, -1)
    amax = np.abs(flat).max(axis=1) if flat.shape[1] else np.zeros(n, np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    y = flat / scale[:, None]
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn)
    codes = codes.view(torch.uint8).numpy().reshape(x.shape)
    return codes, scale


# E2M1 rounding thresholds on |x| (scaled by the block exponent) and whether
# the comparison is strict: at a midpoint the even code wins (round half to
# even), e.g. 0.25 -> 0 (code 0), 0.75 -> 1.0 (code 2), 5.0 -> 4.0 (code 6).
_E2M1_THRESHOLDS = ((0.25, True), (0.75, False), (1.25, True), (1.75, False),
                    (2.5, True), (3.5, False), (5.0, True))


def quantize_mxfp4(x: np.ndarray):
    """MXFP4 along the last axis (a multiple of 32).

    Each 32-element block gets the E8M0 exponent floor(log2(amax)) - 2 (so the
    block maximum lands in [4, 8) before rounding), values are rounded to the
    nearest E2M1 magnitude (ties to the even code) and saturate at 6. Two
    codes per byte, the even element in the low nibble.

    Returns (packed uint8 [..., D/2], scales uint8 [..., D/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    D = x.shape[-1]
    assert D % 32 == 0
    blocks = x.reshape(-1, D // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.maximum(amax, 1e-38))) - 2, 0)
    e = np.clip(e, -127, 127).astype(np.int32)
    scale_bytes = (e + 127).astype(np.uint8)
    y = blocks * np.ldexp(np.float32(1.0), -e)[..., None].astype(np.float32)
    a = np.abs(y)
    c = np.zeros(a.shape, dtype=np.uint8)
    for thr, strict in _E2M1_THRESHOLDS:
        c += (a > thr) if strict else (a >= thr)
    c |= ((y < 0) & (c > 0)).view(np.uint8) << 3
    c = c.reshape(x.shape[:-1] + (D,))
    packed = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    return packed, scale_bytes.reshape(x.shape[:-1] + (D // 32,))


# -------------------------------------------------------------- paged caches

@dataclass
class PagedCache:
    """A key pool in bytes. Row of token slot s in page p starts at
    data[p*page_stride + s*row_stride]; its scale at
    scale[p*scale_page_stride + s*scale_row_stride] (fp32 for FP8, four
    E8M0 bytes for MXFP4). ``scale`` may be a view into ``data``."""
    dtype: int
    data: np.ndarray
    page_stride: int
    row_stride: int
    scale: np.ndarray
    scale_page_stride: int
    scale_row_stride: int
    page_size: int
    num_pages: int
    layout: str = "separate"
    scale_offset: int = -1  # byte offset of scale inside data when shared, else -1


def _alloc_cache(dtype, num_pages, P, D, row_stride, layout, canary):
    if dtype == FP8:
        data_bytes = D
        fill_d = FP8_CANARY if canary else 0
    else:
        data_bytes = D // 2
        fill_d = E2M1_CANARY if canary else 0
    scale_bytes = 4
    if row_stride is None:
        row_stride = data_bytes
    if layout == "separate":
        data = np.full(num_pages * P * row_stride, fill_d, dtype=np.uint8)
        scale = np.zeros(num_pages * P * scale_bytes, dtype=np.uint8)
        if canary:
            if dtype == FP8:
                scale.view(np.uint32)[:] = 0x7FC00000
            else:
                scale[:] = E8M0_CANARY
        return PagedCache(dtype, data, P * row_stride, row_stride, scale,
                          P * scale_bytes, scale_bytes, P, num_pages, layout, -1)
    if layout == "page_block":
        # [P rows of data][P scales] per page
        assert row_stride == data_bytes
        ps = P * (data_bytes + scale_bytes)
        data = np.full(num_pages * ps, fill_d, dtype=np.uint8)
        if canary:
            v = data.reshape(num_pages, ps)[:, P * data_bytes:]
            if dtype == FP8:
                v.reshape(num_pages, P, 4).view(np.uint32)[:] = 0x7FC00000
            else:
                v[:] = E8M0_CANARY
        off = P * data_bytes
        return PagedCache(dtype, data, ps, data_bytes, data[off:], ps, scale_bytes,
                          P, num_pages, layout, off)
    if layout == "row_inline":
        # [data][scale][pad] per row
        assert row_stride >= data_bytes + scale_bytes and row_stride % 4 == 0
        data = np.full(num_pages * P * row_stride, fill_d, dtype=np.uint8)
        if canary:
            v = data.reshape(num_pages * P, row_stride)[:, data_bytes:data_bytes + 4]
            if dtype == FP8:
                v.view(np.uint32)[:] = 0x7FC00000
            else:
                v[:] = E8M0_CANARY
        return PagedCache(dtype, data, P * row_stride, row_stride, data[data_bytes:],
                          P * row_stride, row_stride, P, num_pages, layout, data_bytes)
    raise ValueError("unknown layout %r" % layout)


def _write_rows(cache: PagedCache, rows: np.ndarray, payload: np.ndarray,
                scale_payload: np.ndarray):
    """Store quantized rows at pool row indices ``rows`` (page*P + slot)."""
    P = cache.page_size
    pages, slots = rows // P, rows % P
    nb = payload.shape[1]
    base = pages * cache.page_stride + slots * cache.row_stride
    idx = base[:, None] + np.arange(nb)[None, :]
    cache.data[idx.reshape(-1)] = payload.reshape(-1)
    sb = scale_payload.shape[1]
    if cache.scale_offset >= 0:
        target, off = cache.data, cache.scale_offset
    else:
        target, off = cache.scale, 0
    sbase = off + pages * cache.scale_page_stride + slots * cache.scale_row_stride
    sidx = sbase[:, None] + np.arange(sb)[None, :]
    target[sidx.reshape(-1)] = scale_payload.reshape(-1)


def _quant_keys(dtype, k):
    if dtype == FP8:
        codes, s = quantize_fp8_rows(k)
        return codes, s.view(np.uint8).reshape(-1, 4)
    packed, sc = quantize_mxfp4(k)
    return packed, sc


def _quant_queries(dtype, q):
    """q [R, H, D] → (codes, q_scale) in the library's query layout."""
    if dtype == FP8:
        return quantize_fp8_rows(q)
    return quantize_mxfp4(q)


# ------------------------------------------------------------------ workloads

@dataclass
class DecodeCase:
    name: str
    dtype: int
    H: int
    D: int
    next_n: int
    k: int
    W: int
    q: np.ndarray
    q_scale: np.ndarray
    w: np.ndarray
    cache: PagedCache
    block_tables: np.ndarray
    lens: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return int(self.lens.shape[0])

    @property
    def R(self):
        return self.B * self.next_n


@dataclass
class PrefillCase:
    name: str
    dtype: int
    H: int
    D: int
    k: int
    W: int
    budget_bytes: int
    q: np.ndarray
    q_scale: np.ndarray
    w: np.ndarray
    cache: PagedCache
    block_table: np.ndarray
    visible_end: np.ndarray
    n_keys: int
    meta: dict = field(default_factory=dict)

    @property
    def T(self):
        return int(self.visible_end.shape[0])


def decode_case(lens, *, next_n=1, P=64, dtype=FP8, H=64, D=128, k=2048, W=None,
                pool_pages=None, row_stride=None, layout="separate", seed=0,
                canary=True, bt_width=None, name="decode"):
    """A decode batch: sequence b has lens[b] committed keys in shuffled pages."""
    rng = rng_for(seed)
    lens = np.asarray(lens, dtype=np.int64)
    B = len(lens)
    npg = (lens + P - 1) // P
    need = int(npg.sum())
    if pool_pages is None:
        pool_pages = max(need, int(math.ceil(1.25 * need)), 1)
    assert pool_pages >= need
    if W is None:
        W = int(max(int(lens.max()) if B else 1, 1))
    if bt_width is None:
        bt_width = max(int(npg.max()) if B else 1, 1)
    cache = _alloc_cache(dtype, pool_pages, P, D, row_stride, layout, canary)
    perm = rng.permutation(pool_pages).astype(np.int64)
    bt = np.full((B, bt_width), BT_SENTINEL, dtype=np.int32)
    used = 0
    for b in range(B):
        n = int(npg[b])
        pages = perm[used:used + n]
        used += n
        bt[b, :n] = pages
        L = int(lens[b])
        if L == 0:
            continue
        keys = rng.standard_normal((L, D), dtype=np.float32)
        payload, spay = _quant_keys(dtype, keys)
        rows = (pages[:, None] * P + np.arange(P)[None, :]).reshape(-1)[:L]
        _write_rows(cache, rows, payload, spay)
    R = B * next_n
    qf = rng.standard_normal((R, H, D), dtype=np.float32)
    q, q_scale = _quant_queries(dtype, qf)
    w = (rng.standard_normal((R, H), dtype=np.float32) / np.float32(8.0)).astype(np.float32)
    return DecodeCase(name, dtype, H, D, next_n, k, W, q, q_scale, w, cache, bt,
                      lens.astype(np.int32), {"seed": seed, "pool_pages": pool_pages})


def prefill_case(T, n_keys, *, visible_end=None, P=64, dtype=FP8, H=64, D=128,
                 k=2048, W=None, pool_pages=None, budget_bytes=256_000_000, seed=0,
                 canary=True, name="prefill"):
    """One sequence with n_keys committed keys and T query rows; row r sees
    visible_end[r] keys (default: the compressed-causal rule (r+1)//4)."""
    rng = rng_for(seed)
    if visible_end is None:
        visible_end = np.minimum((np.arange(T, dtype=np.int64) + 1) // 4, n_keys)
    visible_end = np.asarray(visible_end, dtype=np.int32)
    npg = (n_keys + P - 1) // P
    if pool_pages is None:
        pool_pages = max(2 * npg, 1)
    if W is None:
        W = int(max(int(visible_end.max()) if T else 1, 1))
    cache = _alloc_cache(dtype, pool_pages, P, D, None, "separate", canary)
    perm = rng.permutation(pool_pages).astype(np.int64)
    pages = perm[:npg]
    bt = np.full(max(npg, 1), BT_SENTINEL, dtype=np.int32)
    bt[:npg] = pages
    if n_keys:
        keys = rng.standard_normal((n_keys, D), dtype=np.float32)
        payload, spay = _quant_keys(dtype, keys)
        rows = (pages[:, None] * P + np.arange(P)[None, :]).reshape(-1)[:n_keys]
        _write_rows(cache, rows, payload, spay)
    qf = rng.standard_normal((T, H, D), dtype=np.float32)
    q, q_scale = _quant_queries(dtype, qf)
    w = (rng.standard_normal((T, H), dtype=np.float32) / np.float32(8.0)).astype(np.float32)
    return PrefillCase(name, dtype, H, D, k, W, int(budget_bytes), q, q_scale, w, cache,
                       bt, visible_end, int(n_keys), {"seed": seed, "pool_pages": pool_pages})


def mtp_lens(rng, B, forced=(0, 1, 31, 32, 33, 65536)):
    """Length mix of the 32-row-page MTP workload: 1/8 empty, 1/8 a partial
    first page (1..31), 3/4 lognormal with median 8192 (sigma 1) clamped to
    [32, 65536]; the first sequences are forced to the edge lengths."""
    u = rng.random(B)
    part = rng.integers(1, 32, size=B)
    logn = np.clip(np.rint(rng.lognormal(mean=math.log(8192.0), sigma=1.0, size=B)),
                   32, 65536).astype(np.int64)
    lens = np.where(u < 0.125, 0, np.where(u < 0.25, part, logn)).astype(np.int64)
    nf = min(len(forced), B)
    lens[:nf] = np.asarray(forced[:nf])
    return lens


WORKLOADS = {
    1: "single-sequence decode: 1 seq x 4096 keys, FP8, page 64, next_n 1, top-512",
    2: "batched decode: 64 seqs, lens U[1024,32768], FP8, page 64, next_n 1, top-2048, W 65536",
    3: "MTP decode: 128 seqs, next_n 2, FP8, page 32, row stride 144 B, mixed lens, top-2048",
    4: "chunked prefill: 16384 rows over 4096 keys, FP8, page 64, causal (r+1)//4, top-2048",
    5: "MXFP4 decode: 128 seqs, lens U[4096,65536], page 256, next_n 1, top-2048",
}


def workload(i: int, *, seed=None, canary=True, scale_down=1):
    """The five measured workloads at full size (scale_down=1), or a shrunken
    variant with the same structure (lengths divided by scale_down)."""
    if seed is None:
        seed = 1000 + i
    rng = rng_for(seed + 7919)
    s = max(int(scale_down), 1)
    if i == 1:
        return decode_case([4096 // s], next_n=1, P=64, k=512 // min(s, 8), W=4096 // s,
                           pool_pages=max(128 // s, 2), seed=seed, canary=canary,
                           name="w1_single_decode")
    if i == 2:
        B = 64 if s == 1 else max(4, 64 // s)
        lens = rng.integers(1024 // s, 32768 // s + 1, size=B)
        return decode_case(lens, next_n=1, P=64, k=2048 // min(s, 8), W=65536 // s,
                           pool_pages=40000 // s, bt_width=512 // s, seed=seed,
                           canary=canary, name="w2_batched_decode")
    if i == 3:
        B = 128 if s == 1 else max(8, 128 // s)
        lens = mtp_lens(rng, B, forced=(0, 1, 31, 32, 33, 65536 // s))
        if s > 1:
            lens = np.where(lens > 33, np.maximum(lens // s, 34), lens)
        lens = np.minimum(lens, 65536 // s)
        return decode_case(lens, next_n=2, P=32, k=2048 // min(s, 8), W=65536 // s,
                           row_stride=144, bt_width=2048 // s, seed=seed, canary=canary,
                           name="w3_mtp_decode")
    if i == 4:
        T, n_keys = 16384 // s, 4096 // s
        return prefill_case(T, n_keys, P=64, k=2048 // min(s, 8), W=n_keys,
                            pool_pages=max(128 // s, 2),
                            budget_bytes=256_000_000 // (s * s), seed=seed, canary=canary,
                            name="w4_chunked_prefill")
    if i == 5:
        B = 128 if s == 1 else max(8, 128 // s)
        lens = rng.integers(4096 // s, 65536 // s + 1, size=B)
        return decode_case(lens, next_n=1, P=256, dtype=MXFP4, k=2048 // min(s, 8),
                           W=65536 // s, bt_width=256 // s if s <= 256 else 1,
                           seed=seed, canary=canary, name="w5_mxfp4_decode")
    raise ValueError("workload index must be 1..5")


# --------------------------------------------------------- device placement

def to_device(case, device="cuda"):
    """Copy a case's arrays to device tensors (plain uploads). Returns a dict;
    when the cache's scale lives inside its data buffer, ``kscale`` is None and
    ``kscale_offset`` gives its byte offset from ``kdata``."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    c = case.cache
    out = {
        "q": t(case.q),
        "q_scale": None if case.q_scale is None else t(case.q_scale),
        "w": t(case.w),
        "kdata": t(c.data),
        "kscale": None if c.scale_offset >= 0 else t(c.scale),
        "kscale_offset": c.scale_offset,
    }
    if isinstance(case, DecodeCase):
        out["block_tables"] = t(case.block_tables)
        out["lens"] = t(case.lens)
    else:
        out["block_table"] = t(case.block_table)
        out["visible_end"] = t(case.visible_end)
    return out


def ragged_offsets(rng, B, max_q, forced=(0, 1)):
    """Row offsets [B+1] of a ragged decode step: sequence b gets n_b query
    rows drawn from [0, max_q] (the first entries of `forced` and max_q are
    always present when B allows), packed in order."""
    n = rng.integers(0, max_q + 1, size=B)
    for i, v in enumerate(tuple(forced) + (max_q,)):
        if i < B:
            n[i] = min(v, max_q)
    rng.shuffle(n)
    off = np.zeros(B + 1, dtype=np.int32)
    off[1:] = np.cumsum(n)
    return off


# ---------------------------------------------------- sparse MLA over top-k

def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


@dataclass
class MlaCase:
    """Sparse attention inputs: bf16 latent rows (D values) in pages of P
    rows, query rows (bits, [R, H, D]), per-row selected token lists."""
    q: np.ndarray            # uint16 [R, H, D]
    data: np.ndarray         # uint8 pool, num_pages * page_stride bytes
    page_stride: int
    row_stride: int
    page_size: int
    num_pages: int
    block_tables: np.ndarray # int32 [B, bt_stride]
    lens: np.ndarray         # int32 [B] context lengths
    next_n: int
    indices: np.ndarray      # int32 [R, k], -1 past each row's count
    topk_lens: np.ndarray    # int32 [R]
    k: int
    H: int = 64
    D: int = 512

    @property
    def R(self):
        return int(self.q.shape[0])


def mla_case(lens, *, next_n=1, P=64, k=2048, H=64, D=512, row_stride=None, seed=0,
             full=False, holes=False, ascending=False):
    """Selected lists: each row picks min(k, E_r) distinct tokens of its
    visible window (E_r as in decode) in random order (ascending: in
    increasing token order, as the top-k writes them), or every visible token
    when full; holes sets a few entries inside the count to -1."""
    rng = rng_for(seed)
    lens = np.asarray(lens, dtype=np.int64)
    B = len(lens)
    row_stride = row_stride or 2 * D
    npg = (lens + P - 1) // P
    pool = max(int(npg.sum()) + 3, 1)
    perm = rng.permutation(pool).astype(np.int64)
    bt_w = max(int(npg.max()) if B else 1, 1)
    bt = np.full((B, bt_w), BT_SENTINEL, dtype=np.int32)
    data = np.zeros(pool * P * row_stride, dtype=np.uint8)
    used = 0
    for b in range(B):
        n = int(npg[b])
        pages = perm[used:used + n]
        used += n
        bt[b, :n] = pages
        L = int(lens[b])
        if L == 0:
            continue
        rows = (pages[:, None] * P + np.arange(P)[None, :]).reshape(-1)[:L]
        vals = rng.standard_normal((L, D), dtype=np.float32)
        bits = _bf16_bits(vals).view(np.uint8).reshape(L, 2 * D)
        view = data.reshape(pool * P, row_stride)
        view[rows, :2 * D] = bits
    R = B * next_n
    q = _bf16_bits(rng.standard_normal((R, H, D), dtype=np.float32) / np.float32(8.0))
    idx = np.full((R, k), -1, dtype=np.int32)
    tl = np.zeros(R, dtype=np.int32)
    for r in range(R):
        b, j = divmod(r, next_n)
        E = max(0, int(lens[b]) - (next_n - 1 - j))
        n = min(k, E)
        sel = np.arange(E) if full else rng.permutation(E)[:n]
        if ascending:
            sel = np.sort(sel)
        if not full:
            idx[r, :n] = sel
        else:
            idx[r, :n] = sel[:n]
        if holes and n > 4:
            idx[r, rng.integers(0, n, size=3)] = -1
        tl[r] = n
    return MlaCase(q, data, P * row_stride, row_stride, P, pool, bt, lens.astype(np.int32),
                   next_n, idx, tl, k, H, D)
