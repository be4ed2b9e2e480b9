"""MI355X (gfx950) sparse-attention indexer: paged FP8/MXFP4 MQA scores and
per-row top-k, as hand-written HIP kernels behind the C ABI in include/idx.h.

``binding`` is the ctypes layer (same names as the C entry points); ``build``
compiles the library. Importing this package does not load the library; the
first call does, and fails loudly if it has not been built.
"""
from .binding import (  # noqa: F401
    EXPORTS, IDX_ERR_HIP, IDX_ERR_INVALID, IDX_ERR_UNSUPPORTED, IDX_ERR_WORKSPACE,
    IDX_FP8_E4M3, IDX_KIN_BF16, IDX_KIN_F32, IDX_MXFP4, IDX_OK, IDX_QUERY_FILL_NEG_INF, IdxError,
    KVCache, MlaCache, Query,
    idx_build_schedule, idx_kv_cache_write,
    idx_last_error_message, idx_paged_mqa_logits, idx_paged_mqa_logits_varlen,
    idx_prefill_chunked_topk, idx_prefill_chunked_topk_noalloc,
    idx_prefill_rows_per_chunk, idx_prefill_schedule_ints, idx_prefill_scratch_bytes,
    idx_quantize_query, idx_recommended_ctas, idx_recommended_decode_ctas, idx_schedule_ints, idx_sparse_mla_decode,
    idx_sparse_mla_workspace_size, idx_topk,
    idx_topk_workspace_size, idx_validate_decode, idx_varlen_windows, idx_version,
    load, make_kv_cache, make_mla_cache, make_query, ptr, stream_handle,
)
