"""The C ABI without a GPU: the library loads, exports what include/idx.h
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import json
import os
import re
import subprocess

import pytest

import sparse_attention_indexer_page_amd as idx
from sparse_attention_indexer_page_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "idx.h")


@pytest.fixture(scope="module")
def lib():
    from sparse_attention_indexer_page_amd import build
    build.ensure_built()
    return idx.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(idx_[a-z_0-9]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_exactly_the_bound_functions():
    assert _declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_header_compiles_as_plain_c():
    src = '#include "idx.h"\nint main(void){ idx_query q; idx_kv_cache kv; (void)q; (void)kv; return 0; }\n'
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only",
                          "-I", os.path.dirname(HEADER), "-x", "c", "-"],
                         input=src, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_struct_layouts_match_header():
    assert ctypes.sizeof(binding.Query) == 40
    assert ctypes.sizeof(binding.KVCache) == 64
    src = ('#include "idx.h"\n#include <stddef.h>\n'
           '_Static_assert(sizeof(idx_query) == 40, "q");\n'
           '_Static_assert(sizeof(idx_kv_cache) == 64, "kv");\n'
           '_Static_assert(offsetof(idx_kv_cache, scale) == 40, "kv scale");\n'
           '_Static_assert(offsetof(idx_query, weights) == 32, "w");\n')
    res = subprocess.run(["gcc", "-std=c11", "-fsyntax-only", "-I", os.path.dirname(HEADER),
                          "-x", "c", "-"], input=src, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_status_strings_and_version(lib):
    assert lib.idx_status_string(0) == b"IDX_OK"
    assert lib.idx_status_string(3) == b"IDX_ERR_WORKSPACE"
    assert idx.idx_version() >= 100


def _q(dtype=1, heads=64, dim=128, q=0x1000, qs=0x2000, w=0x3000):
    return binding.Query(dtype, heads, dim, 0, q, qs, w)


def _kv(dtype=1, P=64, pages=10, data=0x10000, ps=64 * 128, rs=128, scale=0x20000, sps=256, srs=4):
    return binding.KVCache(dtype, P, pages, data, ps, rs, scale, sps, srs)


def _logits(q, kv, bt=0x4000, bts=8, lens=0x5000, B=2, n=1, cta=0x6000, nc=4, out=0x7000, W=512):
    return idx.load().idx_paged_mqa_logits(ctypes.byref(q), ctypes.byref(kv), bt, bts, lens, B, n,
                                           cta, nc, out, W, None)


@pytest.mark.parametrize("mutate,status", [
    (dict(heads=32), idx.IDX_ERR_UNSUPPORTED),
    (dict(dim=64), idx.IDX_ERR_UNSUPPORTED),
    (dict(dtype=7), idx.IDX_ERR_UNSUPPORTED),
    (dict(q=0), idx.IDX_ERR_INVALID),
    (dict(q=0x1001), idx.IDX_ERR_INVALID),
    (dict(w=0), idx.IDX_ERR_INVALID),
])
def test_logits_rejects_bad_query(lib, mutate, status):
    assert _logits(_q(**mutate), _kv()) == status
    assert idx.idx_last_error_message() != ""


@pytest.mark.parametrize("mutate,status", [
    (dict(P=48), idx.IDX_ERR_INVALID),
    (dict(P=128), idx.IDX_ERR_INVALID),
    (dict(rs=136), idx.IDX_ERR_INVALID),
    (dict(rs=112), idx.IDX_ERR_INVALID),
    (dict(data=0), idx.IDX_ERR_INVALID),
    (dict(scale=0x20002), idx.IDX_ERR_INVALID),
    (dict(ps=64 * 128 - 16), idx.IDX_ERR_INVALID),
    (dict(dtype=2), idx.IDX_ERR_UNSUPPORTED),
    (dict(pages=0), idx.IDX_ERR_INVALID),
])
def test_logits_rejects_bad_cache(lib, mutate, status):
    assert _logits(_q(), _kv(**mutate)) == status


@pytest.mark.parametrize("kw,status", [
    (dict(n=0), idx.IDX_ERR_INVALID), (dict(n=5), idx.IDX_ERR_INVALID),
    (dict(B=0), idx.IDX_ERR_INVALID), (dict(B=16001), idx.IDX_ERR_INVALID),
    (dict(cta=0, B=1025), idx.IDX_ERR_INVALID),  # no schedule buffer: B <= 1024 only
    (dict(nc=0), idx.IDX_ERR_INVALID),
    (dict(W=0), idx.IDX_ERR_INVALID), (dict(W=(1 << 22) + 1), idx.IDX_ERR_INVALID),
    (dict(bts=0), idx.IDX_ERR_INVALID),
])
def test_logits_rejects_bad_shapes(lib, kw, status):
    assert _logits(_q(), _kv(), **kw) == status


def test_mxfp4_query_needs_scales(lib):
    assert _logits(_q(dtype=2, qs=0), _kv(dtype=2, ps=64 * 64, rs=64)) == idx.IDX_ERR_INVALID


@pytest.mark.parametrize("args,status", [
    ((0, 4, 1, 64, 8, 0x100), idx.IDX_ERR_INVALID),
    ((0x100, 0, 1, 64, 8, 0x100), idx.IDX_ERR_INVALID),
    ((0x100, 4, 1, 96, 8, 0x100), idx.IDX_ERR_INVALID),
    ((0x100, 4, 1, 64, 0, 0x100), idx.IDX_ERR_INVALID),
    ((0x100, 4, 9, 64, 8, 0x100), idx.IDX_ERR_INVALID),
    ((0x100, 4, 1, 64, 8, 0), idx.IDX_ERR_INVALID),
])
def test_schedule_rejects_bad_arguments(lib, args, status):
    assert lib.idx_build_schedule(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((0, 512, 0x100, 2, 1, 16, 0x200, None, None, 0), idx.IDX_ERR_INVALID),
    ((0x100, 512, 0x100, 2, 1, 0, 0x200, None, None, 0), idx.IDX_ERR_INVALID),
    ((0x100, 0, 0x100, 2, 1, 16, 0x200, None, None, 0), idx.IDX_ERR_INVALID),
    ((0x100, 65537, 0x100, 2, 1, 16, 0x200, None, None, 0), idx.IDX_ERR_UNSUPPORTED),
])
def test_topk_rejects_bad_arguments(lib, args, status):
    assert lib.idx_topk(*args, None) == status


def test_recommended_decode_ctas_rejects_unsupported_values():
    # unsupported dtype, page size or next_n give 0 before any device query
    assert idx.idx_recommended_decode_ctas(64, 7, 64, 1) == 0
    assert idx.idx_recommended_decode_ctas(64, 1, 48, 1) == 0
    assert idx.idx_recommended_decode_ctas(64, 1, 64, 5) == 0


def test_schedule_buffer_size():
    assert idx.idx_schedule_ints(512) == 2 * 513
    assert idx.idx_schedule_ints(0) == 0


def test_prefill_chunk_rule_reproduces_the_pages_buffer_sizes():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "prefill_width_rule.json")))
    T = g["rows"]
    big = 1 << 62
    # Without a budget limit the scratch is the whole [T, W] buffer.
    full_model = 4 * T * g["model_max_width"]
    right = idx.idx_prefill_scratch_bytes(T, g["right_sized_width"], big)
    assert round(full_model / 1e9) == g["model_max_bytes_approx_gb"]
    assert right == 4 * T * g["right_sized_width"]
    assert round(right / 1e6) == g["right_sized_bytes_approx_mb"]
    # The decimal 256 MB budget of the chunked-prefill workload forces two
    # chunks (at most 15625 rows each); the rows are spread evenly over them,
    # 8192 + 8192, so the scratch holds 8192 rows.
    rows = idx.idx_prefill_rows_per_chunk(4096, 256_000_000)
    assert rows == 15625 and -(-T // rows) == 2
    assert idx.idx_prefill_scratch_bytes(T, 4096, 256_000_000) == 4 * 4096 * 8192
    # Uneven counts: 3 chunks of at most 5 rows for 11 rows -> 4 rows each.
    assert idx.idx_prefill_scratch_bytes(11, 4096, 4 * 4096 * 5) == 4 * 4096 * 4
    # One schedule per chunk, each for min(256, ceil(rows / 15)) work groups.
    assert idx.idx_prefill_schedule_ints(T, 4096, 256_000_000) == 2 * idx.idx_schedule_ints(256)
    assert idx.idx_prefill_schedule_ints(5, 4096, 1) == 5 * idx.idx_schedule_ints(1)
    assert idx.idx_prefill_schedule_ints(T, 4096, big) == idx.idx_schedule_ints(256)
    assert idx.idx_prefill_schedule_ints(1000, 4096, big) == idx.idx_schedule_ints(67)
    # One row per chunk at a budget below one row.
    assert idx.idx_prefill_rows_per_chunk(4096, 1) == 1


@pytest.mark.parametrize("args,want", [
    ((0, 4, 0x200, 8, 64, 10, 100, 0x300), "INVALID"),          # null lens
    ((0x100, 4, 0x200, 8, 48, 10, 100, 0x300), "INVALID"),      # page size
    ((0x100, 16001, 0x200, 8, 64, 10, 100, 0x300), "INVALID"),  # B
    ((0x100, 4, 0x200, 0, 64, 10, 100, 0x300), "INVALID"),      # bt_stride
    ((0x100, 4, 0x200, 8, 64, 0, 100, 0x300), "INVALID"),       # num_pages
    ((0x100, 4, 0x200, 8, 64, 10, -1, 0x300), "INVALID"),       # W
    ((0x100, 4, 0x200, 8, 64, 10, 100, 0x302), "INVALID"),      # result alignment
])
def test_validate_decode_rejects_bad_arguments(lib, args, want):
    assert lib.idx_validate_decode(*args, None) == getattr(idx, "IDX_ERR_" + want)


def test_prefill_rejects_small_scratch(lib):
    q, kv = _q(), _kv()
    rc = lib.idx_prefill_chunked_topk(ctypes.byref(q), ctypes.byref(kv), 0x100, 0x200, 64, 256,
                                      1 << 20, 16, 0, 0x300, 16, 0x400, 1 << 20, 0x500, None)
    assert rc == idx.IDX_ERR_WORKSPACE
    rc = lib.idx_prefill_chunked_topk(ctypes.byref(q), ctypes.byref(kv), 0x100, 0x200, 64, 256,
                                      1 << 20, 16, 0, 0x300, 1 << 30, 0x400, 2, 0x500, None)
    assert rc == idx.IDX_ERR_WORKSPACE


@pytest.mark.parametrize("base", [-1, (1 << 31) - 256])
def test_prefill_rejects_bad_index_base(lib, base):
    q, kv = _q(), _kv()
    rc = lib.idx_prefill_chunked_topk(ctypes.byref(q), ctypes.byref(kv), 0x100, 0x200, 64, 256,
                                      1 << 20, 16, base, 0x300, 1 << 30, 0x400, 1 << 20, 0x500,
                                      None)
    assert rc == idx.IDX_ERR_INVALID


def _kvw(k=0x8000, kd=0, ld=128, N=4, sm=0x9000, kv=None):
    kv = kv if kv is not None else _kv()
    return idx.load().idx_kv_cache_write(k, kd, ld, N, sm, ctypes.byref(kv), None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), idx.IDX_ERR_INVALID),
    (dict(sm=0), idx.IDX_ERR_INVALID),
    (dict(kd=2), idx.IDX_ERR_INVALID),
    (dict(ld=127), idx.IDX_ERR_INVALID),
    (dict(N=-1), idx.IDX_ERR_INVALID),
    (dict(k=0x8004), idx.IDX_ERR_INVALID),          # fp32 pairs need 8-byte alignment
    (dict(k=0x8002, kd=1), idx.IDX_ERR_INVALID),    # bf16 pairs need 4-byte alignment
    (dict(ld=129), idx.IDX_ERR_INVALID),            # odd row stride
    (dict(sm=0x9004), idx.IDX_ERR_INVALID),         # int64 slots need 8-byte alignment
    (dict(kv=_kv(dtype=7)), idx.IDX_ERR_UNSUPPORTED),
    (dict(kv=_kv(P=48)), idx.IDX_ERR_INVALID),
    (dict(kv=_kv(data=0)), idx.IDX_ERR_INVALID),
    (dict(kv=_kv(rs=112)), idx.IDX_ERR_INVALID),
])
def test_kv_write_rejects_bad_arguments(lib, kw, status):
    assert _kvw(**kw) == status
    assert idx.idx_last_error_message() != ""


def test_kv_write_of_no_rows_is_a_no_op(lib):
    # N = 0 launches nothing, so it succeeds without touching the (fake) pointers
    assert _kvw(k=0, sm=0, N=0) == idx.IDX_OK
    assert _kvw(k=0x8002, kd=1, N=0) == idx.IDX_OK


def _qq(x=0x8000, xd=0, ld=8192, R=4, w=0x9000, c=1.0, out=None, dtype=idx.IDX_FP8_E4M3,
        qs=0xA000):
    out = out if out is not None else idx.Query(dtype, 64, 128, 0, 0xB000, qs, 0xC000)
    return idx.load().idx_quantize_query(x, xd, ld, R, w, c, ctypes.byref(out), None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), idx.IDX_ERR_INVALID),
    (dict(w=0), idx.IDX_ERR_INVALID),
    (dict(xd=2), idx.IDX_ERR_INVALID),
    (dict(ld=8191), idx.IDX_ERR_INVALID),
    (dict(ld=8196), idx.IDX_ERR_INVALID),           # rows read eight values at a time
    (dict(x=0x8008), idx.IDX_ERR_INVALID),          # x needs 16-byte alignment
    (dict(w=0x9002), idx.IDX_ERR_INVALID),
    (dict(R=-1), idx.IDX_ERR_INVALID),
    (dict(c=float("inf")), idx.IDX_ERR_INVALID),
    (dict(c=float("nan")), idx.IDX_ERR_INVALID),
    (dict(dtype=5), idx.IDX_ERR_UNSUPPORTED),
    (dict(dtype=idx.IDX_MXFP4, qs=0), idx.IDX_ERR_INVALID),  # MXFP4 scales have nowhere to fold
    (dict(out=idx.Query(1, 32, 128, 0, 0xB000, 0, 0xC000)), idx.IDX_ERR_UNSUPPORTED),
    (dict(out=idx.Query(1, 64, 128, 0, 0xB008, 0, 0xC000)), idx.IDX_ERR_INVALID),
    (dict(out=idx.Query(1, 64, 128, 0, 0xB000, 0, 0)), idx.IDX_ERR_INVALID),
])
def test_quantize_query_rejects_bad_arguments(lib, kw, status):
    assert _qq(**kw) == status
    assert idx.idx_last_error_message() != ""


def test_quantize_query_of_no_rows_is_a_no_op(lib):
    assert _qq(x=0, w=0, R=0) == idx.IDX_OK
    assert _qq(R=0, out=idx.Query(1, 64, 128, 0, 0, 0, 0)) == idx.IDX_OK


def test_varlen_entry_points_reject_bad_arguments(lib):
    q, kv = _q(), _kv()
    L = idx.load()
    # row_offsets null / misaligned
    assert L.idx_paged_mqa_logits_varlen(ctypes.byref(q), ctypes.byref(kv), 0x4000, 8, 0x5000, 0,
                                         2, 2, 0x6000, 4, 0x7000, 512, None) == idx.IDX_ERR_INVALID
    assert L.idx_paged_mqa_logits_varlen(ctypes.byref(q), ctypes.byref(kv), 0x4000, 8, 0x5000,
                                         0x8002, 2, 2, 0x6000, 4, 0x7000, 512,
                                         None) == idx.IDX_ERR_INVALID
    # max_q outside [1, 4]
    assert L.idx_paged_mqa_logits_varlen(ctypes.byref(q), ctypes.byref(kv), 0x4000, 8, 0x5000,
                                         0x8000, 2, 5, 0x6000, 4, 0x7000, 512,
                                         None) == idx.IDX_ERR_INVALID
    assert L.idx_varlen_windows(0x5000, 0x8000, 2, 0, 0x9000, None) == idx.IDX_ERR_INVALID
    assert L.idx_varlen_windows(0x5000, 0x8000, 2, 5, 0x9000, None) == idx.IDX_ERR_INVALID
    assert L.idx_varlen_windows(0, 0x8000, 2, 2, 0x9000, None) == idx.IDX_ERR_INVALID
    assert L.idx_varlen_windows(0x5000, 0x8000, 0, 2, 0x9000, None) == idx.IDX_ERR_INVALID
    assert L.idx_varlen_windows(0x5000, 0x8000, 16001, 2, 0x9000, None) == idx.IDX_ERR_INVALID
    assert L.idx_varlen_windows(0x5002, 0x8000, 2, 2, 0x9000, None) == idx.IDX_ERR_INVALID
    assert idx.idx_last_error_message() != ""


@pytest.mark.parametrize("flags", [2, 0x80000000 - (1 << 32), 3])
def test_logits_rejects_unknown_query_flags(lib, flags):
    q = binding.Query(1, 64, 128, flags, 0x1000, 0x2000, 0x3000)
    assert _logits(q, _kv()) == idx.IDX_ERR_INVALID
    assert "flags" in idx.idx_last_error_message()


def test_sparse_mla_rejects_bad_arguments(lib):
    L = idx.load()
    kv = idx.MlaCache(64, 0, 10, 0x10000, 64 * 1024, 1024)
    def call(q=0x1000, kv=kv, bt=0x2000, bts=8, B=2, n=1, ind=0x3000, tl=0x4000, k=16, scale=0.1,
             out=0x5000, lse=0, ws=0x6000, wsb=1 << 30):
        return L.idx_sparse_mla_decode(q, ctypes.byref(kv), bt, bts, B, n, ind, tl, k, scale, out,
                                       lse, ws, wsb, None)
    assert call(q=0) == idx.IDX_ERR_INVALID
    assert call(kv=idx.MlaCache(48, 0, 10, 0x10000, 64 * 1024, 1024)) == idx.IDX_ERR_INVALID
    assert call(kv=idx.MlaCache(64, 0, 10, 0x10000, 64 * 1024, 1008)) == idx.IDX_ERR_INVALID
    assert call(kv=idx.MlaCache(64, 0, 10, 0x10000, 1024, 1024)) == idx.IDX_ERR_INVALID
    assert call(n=5) == idx.IDX_ERR_INVALID
    assert call(k=0) == idx.IDX_ERR_INVALID
    assert call(scale=float("inf")) == idx.IDX_ERR_INVALID
    assert call(q=0x1008) == idx.IDX_ERR_INVALID
    assert call(wsb=16) == idx.IDX_ERR_WORKSPACE
    assert idx.idx_sparse_mla_workspace_size(2, 16) == 2 * 1 * 64 * 514 * 4
    assert idx.idx_sparse_mla_workspace_size(0, 16) == 0


def _topk_loads(E, NT, IPT, wave_kernel):
    """The top-k kernels' row loads as (byte offset, read by the kernel)
    pairs: the block kernel gives wave w of NT/64 the indices
    [w*rounds*64, ...), lane l of item i index base + 64 i + l, and keeps the
    item iff i < rounds and 64 i < E - base - l; the one-wave kernel keeps
    item i of lane l iff 64 i < E - l. The byte offset is the load's vector
    offset (the item step folded in), which the buffer bound of E*4 bytes
    checks."""
    loads = []
    NW = 1 if wave_kernel else NT // 64
    rounds = IPT if wave_kernel else (E + NW * 64 - 1) // (NW * 64)
    for w in range(NW):
        base = w * rounds * 64
        for lane in range(64):
            left = E - base - lane
            for i in range(IPT):
                off = (base + lane) * 4 + 256 * i
                keep = (64 * i < left) if wave_kernel else (i < rounds and 64 * i < left)
                loads.append((off, keep))
    return loads


@pytest.mark.parametrize("wave_kernel,NT,buckets", [
    (False, 1024, [(4, 4096), (8, 8192), (16, 16384), (32, 32768), (64, 65536)]),
    (True, 64, [(16, 1024), (32, 2048), (64, 4096)]),
])
def test_topk_row_loads_stay_inside_the_row(wave_kernel, NT, buckets):
    """Every load the top-k kernels keep lies inside the row's E scores, so
    every load past the row (offset >= E*4, which the buffer bound turns into
    a zero without touching memory) is one the kernel discards; the kept
    loads cover each index below E exactly once."""
    for IPT, max_e in buckets:
        for E in sorted({1, 63, 64, 65, max_e // 2 + 1, max_e - 1, max_e}):
            if E < 1 or E > max_e:
                continue
            seen = [0] * E
            for off, keep in _topk_loads(E, NT, IPT, wave_kernel):
                if keep:
                    assert off + 4 <= 4 * E, (IPT, E, off)
                    seen[off // 4] += 1
            assert all(c == 1 for c in seen), (IPT, E)


def test_prefill_noalloc_rejects_plans_beyond_its_fixed_scratch(lib):
    """The no-allocation prefill checks on the host, before any HIP call, that
    the chunk plan fits its fixed scratch: at W = 65536 the 64 MiB logits
    cap allows 256 rows per chunk, and 2000000 rows then need 7813 schedules
    of 18 work groups (38 entries each), more than the 2^18 entries it
    holds (1765888 rows fit)."""
    q, kv = _q(), _kv()
    fake = ctypes.c_void_p(0x10000)
    st = lib.idx_prefill_chunked_topk_noalloc(ctypes.byref(q), ctypes.byref(kv), fake, fake,
                                              2000000, 65536, 1 << 40, 2048, 0, fake, None)
    assert st == idx.IDX_ERR_WORKSPACE
    assert b"fixed scratch" in lib.idx_last_error()
    for T, W, status in ((0, 4096, idx.IDX_ERR_INVALID), (10, 0, idx.IDX_ERR_INVALID),
                         (10, 65537, idx.IDX_ERR_UNSUPPORTED)):
        assert lib.idx_prefill_chunked_topk_noalloc(ctypes.byref(q), ctypes.byref(kv), fake, fake,
                                                    T, W, 1 << 30, 16, 0, fake, None) == status


def test_noalloc_capacities_match_the_header():
    text = open(HEADER).read()
    logits = re.search(r"#define IDX_NOALLOC_LOGITS_BYTES \((\d+)ll << (\d+)\)", text)
    ints = re.search(r"#define IDX_NOALLOC_SCHEDULE_INTS \((\d+)ll << (\d+)\)", text)
    assert int(logits.group(1)) << int(logits.group(2)) == binding.IDX_NOALLOC_LOGITS_BYTES
    assert int(ints.group(1)) << int(ints.group(2)) == binding.IDX_NOALLOC_SCHEDULE_INTS
