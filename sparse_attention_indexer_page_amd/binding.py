"""ctypes binding of libidx.so (include/idx.h), argument marshalling only.

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: tensors become device pointers, streams become
hipStream_t handles, and a non-zero status becomes an ``IdxError``. The
library must have been built (``sparse_attention_indexer_page_amd.build``);
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libidx.so")

IDX_OK = 0
IDX_ERR_INVALID = 1
IDX_ERR_UNSUPPORTED = 2
IDX_ERR_WORKSPACE = 3
IDX_ERR_HIP = 4

IDX_FP8_E4M3 = 1
IDX_MXFP4 = 2

IDX_QUERY_FILL_NEG_INF = 1

# capacity of the fixed scratch of idx_prefill_chunked_topk_noalloc
IDX_NOALLOC_LOGITS_BYTES = 64 << 20
IDX_NOALLOC_SCHEDULE_INTS = 1 << 18
IDX_KIN_F32 = 0
IDX_KIN_BF16 = 1

# Every symbol include/idx.h declares.
EXPORTS = (
    "idx_schedule_ints", "idx_recommended_ctas", "idx_recommended_decode_ctas", "idx_build_schedule",
    "idx_paged_mqa_logits", "idx_paged_mqa_logits_varlen", "idx_varlen_windows",
    "idx_topk_workspace_size", "idx_topk",
    "idx_prefill_rows_per_chunk", "idx_prefill_scratch_bytes",
    "idx_prefill_schedule_ints", "idx_prefill_chunked_topk", "idx_prefill_chunked_topk_noalloc",
    "idx_kv_cache_write",
    "idx_quantize_query", "idx_sparse_mla_workspace_size", "idx_sparse_mla_decode",
    "idx_validate_decode", "idx_status_string", "idx_last_error", "idx_version",
)


class MlaCache(ctypes.Structure):
    _fields_ = [("page_size", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("num_pages", ctypes.c_int64), ("data", ctypes.c_void_p),
                ("page_stride_bytes", ctypes.c_int64), ("row_stride_bytes", ctypes.c_int64)]


class IdxError(RuntimeError):
    def __init__(self, status: int, func: str, message: str):
        self.status = status
        super().__init__("%s failed (%s): %s" % (func, _status_name(status), message))


class Query(ctypes.Structure):
    """struct idx_query."""
    _fields_ = [("dtype", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("q_scale", ctypes.c_void_p),
                ("weights", ctypes.c_void_p)]


class KVCache(ctypes.Structure):
    """struct idx_kv_cache."""
    _fields_ = [("dtype", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int64), ("data", ctypes.c_void_p),
                ("page_stride_bytes", ctypes.c_int64), ("row_stride_bytes", ctypes.c_int64),
                ("scale", ctypes.c_void_p), ("scale_page_stride_bytes", ctypes.c_int64),
                ("scale_row_stride_bytes", ctypes.c_int64)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libidx.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            "libidx.so is not built (%s); build it with "
            "sparse_attention_indexer_page_amd.build.build()" % path)
    try:  # bind the HIP runtime torch already uses, so its streams are valid here
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    st = ctypes.c_int
    sig = {
        "idx_schedule_ints": (i64, [i32]),
        "idx_recommended_ctas": (i32, [i32]),
        "idx_recommended_decode_ctas": (i32, [i32, i32, i32, i32]),
        "idx_build_schedule": (st, [P, i32, i32, i32, i32, P, P]),
        "idx_paged_mqa_logits": (st, [ctypes.POINTER(Query), ctypes.POINTER(KVCache), P, i64,
                                      P, i32, i32, P, i32, P, i64, P]),
        "idx_paged_mqa_logits_varlen": (st, [ctypes.POINTER(Query), ctypes.POINTER(KVCache), P,
                                             i64, P, P, i32, i32, P, i32, P, i64, P]),
        "idx_varlen_windows": (st, [P, P, i32, i32, P, P]),
        "idx_topk_workspace_size": (sz, [i32, i64, i32]),
        "idx_topk": (st, [P, i64, P, i32, i32, i32, P, P, P, sz, P]),
        "idx_prefill_rows_per_chunk": (i64, [i64, i64]),
        "idx_prefill_scratch_bytes": (i64, [i32, i64, i64]),
        "idx_prefill_schedule_ints": (i64, [i32, i64, i64]),
        "idx_prefill_chunked_topk": (st, [ctypes.POINTER(Query), ctypes.POINTER(KVCache), P, P,
                                          i32, i64, i64, i32, i32, P, i64, P, i64, P, P]),
        "idx_prefill_chunked_topk_noalloc": (st, [ctypes.POINTER(Query), ctypes.POINTER(KVCache),
                                                  P, P, i32, i64, i64, i32, i32, P, P]),
        "idx_kv_cache_write": (st, [P, i32, i64, i32, P, ctypes.POINTER(KVCache), P]),
        "idx_quantize_query": (st, [P, i32, i64, i32, P, ctypes.c_float,
                                    ctypes.POINTER(Query), P]),
        "idx_sparse_mla_workspace_size": (sz, [i32, i32]),
        "idx_sparse_mla_decode": (st, [P, ctypes.POINTER(MlaCache), P, i64, i32, i32, P, P, i32,
                                       ctypes.c_float, P, P, P, sz, P]),
        "idx_validate_decode": (st, [P, i32, P, i64, i32, i64, i64, P, P]),
        "idx_status_string": (ctypes.c_char_p, [st]),
        "idx_last_error": (ctypes.c_char_p, []),
        "idx_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _status_name(status: int) -> str:
    try:
        return load().idx_status_string(status).decode()
    except Exception:  # library not loadable: plain number
        return str(status)


def _check(status: int, func: str):
    if status != IDX_OK:
        raise IdxError(status, func, load().idx_last_error().decode())


def ptr(x) -> int | None:
    """Device pointer of a tensor (or an int address passed through)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def stream_handle(stream) -> int | None:
    """hipStream_t of a torch stream (None: torch's current stream)."""
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_query(dtype, q, q_scale, weights, num_heads=64, head_dim=128, flags=0) -> Query:
    return Query(dtype, num_heads, head_dim, flags, ptr(q), ptr(q_scale), ptr(weights))


def make_kv_cache(dtype, page_size, num_pages, data, page_stride_bytes, row_stride_bytes,
                  scale, scale_page_stride_bytes, scale_row_stride_bytes) -> KVCache:
    return KVCache(dtype, page_size, num_pages, ptr(data), page_stride_bytes, row_stride_bytes,
                   ptr(scale), scale_page_stride_bytes, scale_row_stride_bytes)


# ------------------------------------------------------------ entry points

def idx_version() -> int:
    return load().idx_version()


def idx_schedule_ints(n_ctas: int) -> int:
    return load().idx_schedule_ints(n_ctas)


def idx_recommended_ctas(rows: int) -> int:
    return load().idx_recommended_ctas(rows)


def idx_recommended_decode_ctas(rows: int, dtype: int, page_size: int, next_n: int) -> int:
    return load().idx_recommended_decode_ctas(rows, dtype, page_size, next_n)


def idx_validate_decode(context_lens, B, block_tables, bt_stride, page_size, num_pages, W, result,
                        stream=None):
    _check(load().idx_validate_decode(ptr(context_lens), B, ptr(block_tables), bt_stride, page_size,
                                      num_pages, W, ptr(result), stream_handle(stream)),
           "idx_validate_decode")


def idx_build_schedule(context_lens, B, next_n, page_size, n_ctas, cta_info, stream=None):
    _check(load().idx_build_schedule(ptr(context_lens), B, next_n, page_size, n_ctas,
                                     ptr(cta_info), stream_handle(stream)),
           "idx_build_schedule")


def idx_paged_mqa_logits(query: Query, kv: KVCache, block_tables, bt_stride, context_lens, B,
                         next_n, cta_info, n_ctas, logits, W, stream=None):
    _check(load().idx_paged_mqa_logits(ctypes.byref(query), ctypes.byref(kv), ptr(block_tables),
                                       bt_stride, ptr(context_lens), B, next_n, ptr(cta_info),
                                       n_ctas, ptr(logits), W, stream_handle(stream)),
           "idx_paged_mqa_logits")


def idx_topk_workspace_size(rows, W, k) -> int:
    return load().idx_topk_workspace_size(rows, W, k)


def idx_topk(logits, W, context_lens, B, next_n, k, out_idx, out_count=None, ws=None,
             ws_bytes=0, stream=None):
    _check(load().idx_topk(ptr(logits), W, ptr(context_lens), B, next_n, k, ptr(out_idx),
                           ptr(out_count), ptr(ws), ws_bytes, stream_handle(stream)),
           "idx_topk")


def idx_prefill_rows_per_chunk(W, budget_bytes) -> int:
    return load().idx_prefill_rows_per_chunk(W, budget_bytes)


def idx_prefill_scratch_bytes(T, W, budget_bytes) -> int:
    return load().idx_prefill_scratch_bytes(T, W, budget_bytes)


def idx_prefill_schedule_ints(T, W, budget_bytes) -> int:
    return load().idx_prefill_schedule_ints(T, W, budget_bytes)


def idx_prefill_chunked_topk(query: Query, kv: KVCache, block_table, visible_end, T, W,
                             budget_bytes, k, index_base, logits_scratch, scratch_bytes,
                             cta_scratch, cta_scratch_ints, out_idx, stream=None):
    _check(load().idx_prefill_chunked_topk(ctypes.byref(query), ctypes.byref(kv),
                                           ptr(block_table), ptr(visible_end), T, W,
                                           budget_bytes, k, index_base, ptr(logits_scratch),
                                           scratch_bytes,
                                           ptr(cta_scratch), cta_scratch_ints, ptr(out_idx),
                                           stream_handle(stream)),
           "idx_prefill_chunked_topk")


def idx_prefill_chunked_topk_noalloc(query: Query, kv: KVCache, block_table, visible_end, T, W,
                                     budget_bytes, k, index_base, out_idx, stream=None):
    _check(load().idx_prefill_chunked_topk_noalloc(ctypes.byref(query), ctypes.byref(kv),
                                                   ptr(block_table), ptr(visible_end), T, W,
                                                   budget_bytes, k, index_base, ptr(out_idx),
                                                   stream_handle(stream)),
           "idx_prefill_chunked_topk_noalloc")


def idx_last_error_message() -> str:
    """idx_last_error() of the calling thread."""
    return load().idx_last_error().decode()


def idx_kv_cache_write(k, k_dtype, k_row_stride, N, slot_mapping, kv: KVCache, stream=None):
    _check(load().idx_kv_cache_write(ptr(k), k_dtype, k_row_stride, N, ptr(slot_mapping),
                                     ctypes.byref(kv), stream_handle(stream)),
           "idx_kv_cache_write")


def idx_quantize_query(x, x_dtype, x_row_stride, R, w, c, out: Query, stream=None):
    _check(load().idx_quantize_query(ptr(x), x_dtype, x_row_stride, R, ptr(w), c,
                                     ctypes.byref(out), stream_handle(stream)),
           "idx_quantize_query")


def idx_paged_mqa_logits_varlen(query: Query, kv: KVCache, block_tables, bt_stride,
                                context_lens, row_offsets, B, max_q, cta_info, n_ctas, logits,
                                W, stream=None):
    _check(load().idx_paged_mqa_logits_varlen(
        ctypes.byref(query), ctypes.byref(kv), ptr(block_tables), bt_stride, ptr(context_lens),
        ptr(row_offsets), B, max_q, ptr(cta_info), n_ctas, ptr(logits), W,
        stream_handle(stream)), "idx_paged_mqa_logits_varlen")


def idx_varlen_windows(context_lens, row_offsets, B, max_q, visible_end, stream=None):
    _check(load().idx_varlen_windows(ptr(context_lens), ptr(row_offsets), B, max_q,
                                     ptr(visible_end), stream_handle(stream)),
           "idx_varlen_windows")


def make_mla_cache(page_size, num_pages, data, page_stride_bytes, row_stride_bytes) -> MlaCache:
    return MlaCache(page_size, 0, num_pages, ptr(data), page_stride_bytes, row_stride_bytes)


def idx_sparse_mla_workspace_size(R, k) -> int:
    return load().idx_sparse_mla_workspace_size(R, k)


def idx_sparse_mla_decode(q, kv: MlaCache, block_tables, bt_stride, B, next_n, indices,
                          topk_lens, k, scale, out, lse, ws, ws_bytes, stream=None):
    _check(load().idx_sparse_mla_decode(ptr(q), ctypes.byref(kv), ptr(block_tables), bt_stride,
                                        B, next_n, ptr(indices), ptr(topk_lens), k, scale,
                                        ptr(out), ptr(lse), ptr(ws), ws_bytes,
                                        stream_handle(stream)),
           "idx_sparse_mla_decode")
