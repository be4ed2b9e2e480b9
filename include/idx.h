/*
 * idx.h — C ABI of the MI355X (gfx950) sparse-attention indexer library.
 *
 * The library computes, for every query row of a batch, the indexer scores
 *     logits[r][t] = sum_h w[r][h] * max(0, k_scale[t] * (q[r][h] . k[t]))
 * over a single-head K cache stored in fixed-size physical pages, and then the
 * row's top-k token indices. The pages this is built from name the op
 * "mqa-logits" followed by "indexer_score_topk" (ROCm/ATOM PR #1709 "Add fp4
 * indexer fo dsv4": commit on the single-kernel varctx schedule, commit on the
 * forward_pre / score_topk_from split, commit on right-sizing the prefill
 * logits; vllm-project/DeepGEMM PR #14: summary, "FP8 paged-MQA logits").
 *
 * Conventions shared by every entry point:
 *   - All pointers are device pointers unless the comment says "host".
 *   - The caller owns every buffer. The library never allocates, frees or
 *     synchronizes; work is enqueued asynchronously on `stream` (a
 *     hipStream_t; NULL is the default stream). No call makes a hidden
 *     device-to-host copy, so every entry point can be captured into a HIP
 *     graph (flashinfer PR #3269, review discussion on .item() syncs in the
 *     DSv4 sparse-MLA input checks).
 *   - Argument errors are reported as an idx_status, never by aborting
 *     (flashinfer PR #3269, review: validate with explicit errors, not
 *     asserts). The message of the last failure on the calling thread is in
 *     idx_last_error(). Host-side checks run before any HIP call, so a
 *     rejected call touches no device state.
 *   - Device-side contracts that cannot be checked without a sync
 *     (len <= W, block-table entries of visible tokens naming pages of the
 *     pool) are not checked; K loads are bounds-checked against the pool so a
 *     bad page id reads zeros instead of faulting (ATOM PR #1709, commit on
 *     the ragged-window refresh: a bounds-check-off buffer load turned stale
 *     metadata into a memory fault).
 *   - Supported shapes: num_heads = 64, head_dim = 128, page_size in
 *     {32, 64, 256}, next_n in [1, 4], top-k row width W <= 65536.
 *
 * Thread safety: calls are stateless apart from the thread-local error
 * string; concurrent calls on different streams are safe.
 */
#ifndef IDX_H_
#define IDX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum idx_status {
    IDX_OK = 0,
    IDX_ERR_INVALID = 1,     /* bad pointer, size, stride or alignment */
    IDX_ERR_UNSUPPORTED = 2, /* valid request this library does not implement */
    IDX_ERR_WORKSPACE = 3,   /* caller-provided buffer too small */
    IDX_ERR_HIP = 4          /* a HIP runtime call failed */
} idx_status;

/* Element formats of q and of the K cache. FP8 is OCP E4M3FN (the cache is
 * fp8_e4m3: sglang PR #11993, summary of changes). MXFP4 is OCP E2M1, two
 * values per byte with the even element in the low nibble, plus one E8M0
 * scale byte per 32 consecutive elements; a uint8 cache selects it (ATOM PR
 * #1709, commit on the forward_pre split). */
typedef enum idx_dtype {
    IDX_FP8_E4M3 = 1,
    IDX_MXFP4 = 2
} idx_dtype;

/* Query rows. R rows, H heads, head dim D.
 *   FP8:   q       bytes [R][H][D]
 *          q_scale fp32  [R] (one scale per token), or NULL meaning 1
 *   MXFP4: q       bytes [R][H][D/2]
 *          q_scale E8M0  [R][H][D/32] (required)
 *   weights fp32 [R][H] (per-row, per-head indexer weights; any sign).
 * q must be 16-byte aligned. */
/* Query flag: idx_paged_mqa_logits / idx_paged_mqa_logits_varlen also write
 * -inf to every column [E_r, W) of every row of the logits buffer (E_r = 0
 * for a ragged buffer row no sequence owns), so the whole buffer is defined
 * for a consumer that reads full rows; one more pass over the buffer. The
 * prefill entry and idx_quantize_query ignore it. */
#define IDX_QUERY_FILL_NEG_INF 1

typedef struct idx_query {
    int32_t dtype;     /* idx_dtype */
    int32_t num_heads; /* H; must be 64 */
    int32_t head_dim;  /* D; must be 128 */
    int32_t flags;     /* 0 or IDX_QUERY_FILL_NEG_INF; other bits are rejected */
    const void *q;
    const void *q_scale;
    const float *weights;
} idx_query;

/* Paged single-head K cache. Token slot s of physical page p:
 *   data row  at data  + p*page_stride_bytes       + s*row_stride_bytes
 *   its scale at scale + p*scale_page_stride_bytes + s*scale_row_stride_bytes
 * FP8 rows hold D bytes and the scale is one fp32; MXFP4 rows hold D/2 bytes
 * and the scale is D/32 E8M0 bytes. The two stride pairs express a separate
 * scale array, scales interleaved in a padded row (e.g. 144-byte rows) and
 * per-page [P rows][P scales] blocks (DeepGEMM PR #14 summary: padded page
 * strides; fused-cache API). Data rows must be 16-byte aligned (data,
 * page_stride_bytes, row_stride_bytes multiples of 16); scale addresses
 * 4-byte aligned. num_pages bounds every K load. */
typedef struct idx_kv_cache {
    int32_t dtype;     /* idx_dtype; must equal the query dtype */
    int32_t page_size; /* P: 32, 64 or 256 */
    int64_t num_pages;
    const void *data;
    int64_t page_stride_bytes;
    int64_t row_stride_bytes;
    const void *scale;
    int64_t scale_page_stride_bytes;
    int64_t scale_row_stride_bytes;
} idx_kv_cache;

/* Number of int32 entries of a schedule buffer for n_ctas work groups. */
int64_t idx_schedule_ints(int32_t n_ctas);

/* Number of work groups a schedule should be built for on this device
 * when the batch has `rows` query rows (host only; queries the current
 * device once). Returns a positive count, or 0 when no device is present. */
int32_t idx_recommended_ctas(int32_t rows);

/* Work groups for idx_paged_mqa_logits on this device, by what sets the
 * bytes each of its single-wave work groups keeps in flight: FP8 keys in
 * 64-token blocks (pages of 64 or 256 rows) with one query row per sequence
 * stream 8 KB blocks, and one wave per SIMD (4 per CU) keeps enough of them
 * in flight while no two waves of a SIMD compete for issue; smaller blocks
 * (32-row pages, MXFP4 keys) want two waves per SIMD (8 per CU) where the
 * CU's 160 KB of LDS holds eight of their work groups (up to three query rows
 * per sequence), else 4 per CU, so every work group is resident at once. At
 * least `rows`. Host only; 0 when no device is present or dtype / page_size /
 * next_n are not supported values. */
int32_t idx_recommended_decode_ctas(int32_t rows, int32_t dtype, int32_t page_size,
                                    int32_t next_n);

/*
 * Build the decode work split (ATOM PR #1709, commit on compute_varctx_schedule:
 * one kernel writes the split straight into a fixed-address buffer that a
 * captured graph reads, replacing many small launches). Sequence b holds
 * ceil(context_lens[b] / BK) blocks of BK = min(page_size, 64) tokens, so no
 * block straddles two pages (DeepGEMM PR #14: BLOCK_KV = min(PAGE_KV, 64), a
 * tile must not span two non-contiguous pages). The blocks of all sequences,
 * in order, are split into n_ctas contiguous, near-equal ranges.
 *
 *   context_lens  int32 [B], device; read at kernel time (so a graph replay
 *                 sees the lengths current at replay)
 *   cta_info      int32 [idx_schedule_ints(n_ctas)], device, written: entry c
 *                 holds the (sequence, block) where work group c starts; entry
 *                 n_ctas holds the end (B, 0).
 * Errors: IDX_ERR_INVALID for null pointers, B < 1 or B > 16000,
 * next_n outside [1,4], page_size not 32/64/256, n_ctas < 1 or > 1<<20.
 */
idx_status idx_build_schedule(const int32_t *context_lens, int32_t B, int32_t next_n,
                              int32_t page_size, int32_t n_ctas, int32_t *cta_info,
                              void *stream);

/*
 * Decode scores ("mqa-logits"). Query row r = b*next_n + j (j < next_n) of
 * sequence b sees E_r = max(0, context_lens[b] - (next_n - 1 - j)) tokens;
 * for t < E_r it writes logits[r*W + t]. Columns t >= E_r are not written
 * (unless q->flags has IDX_QUERY_FILL_NEG_INF: then they are set to -inf).
 *
 *   q, kv          descriptors above (host pointers to structs holding
 *                  device pointers); kv->dtype == q->dtype
 *   block_tables   int32 [B][bt_stride]; entry i of row b is the physical page
 *                  of tokens [i*P, (i+1)*P); only entries < ceil(len_b / P)
 *                  are read
 *   cta_info       schedule from idx_build_schedule with the same lens, B,
 *                  next_n, page_size and n_ctas; or NULL when B <= 1024: each
 *                  work group then computes its own range of the same split
 *                  from context_lens (the kernel's internal schedule build,
 *                  which ATOM PR #1709 says a passed cta_info skips), saving
 *                  the builder launch
 *   logits         fp32 [B*next_n][W]
 * Errors: IDX_ERR_INVALID (null pointer, shape, alignment, W outside
 * [1, 2^22], cta_info NULL with B > 1024), IDX_ERR_UNSUPPORTED (H != 64,
 * D != 128, dtype mismatch). Work is split by lengths clamped to 2^22 tokens,
 * so a length breaking the contract len <= W cannot overflow the split.
 */
idx_status idx_paged_mqa_logits(const idx_query *q, const idx_kv_cache *kv,
                                const int32_t *block_tables, int64_t bt_stride,
                                const int32_t *context_lens, int32_t B, int32_t next_n,
                                const int32_t *cta_info, int32_t n_ctas, float *logits,
                                int64_t W, void *stream);

/*
 * Ragged decode (speculative decoding with per-sequence draft counts): the
 * query rows of a step are packed, sequence b owning rows
 * [row_offsets[b], row_offsets[b+1]) -- n_b = row_offsets[b+1] -
 * row_offsets[b] rows, 0 <= n_b <= max_q <= 4 -- and its row j sees
 * E = max(0, context_lens[b] - (n_b - 1 - j)) tokens: each draft row's window
 * ends at its own position (ATOM PR #1709, commits on the ragged varlen
 * windows: the windows move every decode step and a rectangular step is the
 * uniform case n_b = next_n; offsets b*next_n reproduce idx_paged_mqa_logits
 * exactly). Buffers keep the fixed shape of B*max_q rows so a captured graph
 * stays valid whatever the step's draft counts are:
 *   q, weights, q_scale  rows [0, B*max_q); rows >= row_offsets[B] unread
 *   row_offsets          int32 [B+1], device, non-decreasing from 0, read at
 *                        kernel time (offsets outside the contract drop rows;
 *                        they never address outside the B*max_q rows)
 *   cta_info             idx_build_schedule(context_lens, B, max_q, ...), or
 *                        NULL when B <= 1024
 *   logits               fp32 [B*max_q][W]; only rows < row_offsets[B] and
 *                        columns < their E are written
 * Other arguments and errors as idx_paged_mqa_logits (max_q in place of
 * next_n), plus IDX_ERR_INVALID for a null or misaligned row_offsets. A
 * sequence with no rows still costs its scan: pass a 0 length for it.
 */
idx_status idx_paged_mqa_logits_varlen(const idx_query *q, const idx_kv_cache *kv,
                                       const int32_t *block_tables, int64_t bt_stride,
                                       const int32_t *context_lens, const int32_t *row_offsets,
                                       int32_t B, int32_t max_q, const int32_t *cta_info,
                                       int32_t n_ctas, float *logits, int64_t W, void *stream);

/*
 * Per-row visible ends of a ragged decode step, built on the device every
 * step ("compute_varqlen_windows" in ATOM PR #1709: stale windows replayed
 * by a captured graph were the cause of a memory fault there). Writes
 * visible_end[r] for every r < B*max_q: the E of the row's owner as in
 * idx_paged_mqa_logits_varlen, 0 for rows no sequence owns. Then
 * idx_topk(logits, W, visible_end, B*max_q, 1, k, ...) selects per packed
 * row, with empty selections for the unowned rows.
 * Errors: IDX_ERR_INVALID (null or misaligned pointers, B outside [1, 16000],
 * max_q outside [1, 4]).
 */
idx_status idx_varlen_windows(const int32_t *context_lens, const int32_t *row_offsets, int32_t B,
                              int32_t max_q, int32_t *visible_end, void *stream);

/* Workspace bytes idx_topk needs for `rows` rows of width W (0 for W <= 65536). */
size_t idx_topk_workspace_size(int32_t rows, int64_t W, int32_t k);

/*
 * Per-row top-k ("indexer_score_topk"). Row r = b*next_n + j has E_r as in
 * idx_paged_mqa_logits and reads logits[r*W + t] for t < E_r only. It writes
 * the min(k, E_r) token indices with the largest logits to
 * out_idx[r*k .. r*k + k), in ascending index order, padded with -1; equal
 * logits are taken lowest index first, and -0.0 equals +0.0. Indices are
 * sequence-local (ATOM PR #1709, commit on the prefill width: the FP4 path
 * emits seq-local indices). out_count[r] = min(k, E_r) when out_count is not
 * NULL. Logits must be finite for t < E_r.
 * Errors: IDX_ERR_INVALID (null pointer, k < 1, W < 1),
 * IDX_ERR_UNSUPPORTED (W > 65536), IDX_ERR_WORKSPACE (ws_bytes below
 * idx_topk_workspace_size).
 */
idx_status idx_topk(const float *logits, int64_t W, const int32_t *context_lens, int32_t B,
                    int32_t next_n, int32_t k, int32_t *out_idx, int32_t *out_count,
                    void *ws, size_t ws_bytes, void *stream);

/* Rows per prefill chunk for width W under a logits budget of budget_bytes:
 * max(1, floor(budget_bytes / (4*W))) (host only). */
int64_t idx_prefill_rows_per_chunk(int64_t W, int64_t budget_bytes);

/* Logits scratch bytes idx_prefill_chunked_topk needs: 4*W*ceil(T/n), where
 * n = ceil(T / rows per chunk) is the number of chunks the budget requires
 * and the rows are spread evenly over them (host only). */
int64_t idx_prefill_scratch_bytes(int32_t T, int64_t W, int64_t budget_bytes);

/* int32 entries of cta_scratch idx_prefill_chunked_topk needs: one schedule
 * (idx_schedule_ints of the chunk's work-group count) per chunk, all built by
 * one launch before the first chunk is scored. */
int64_t idx_prefill_schedule_ints(int32_t T, int64_t W, int64_t budget_bytes);

/*
 * Prefill: scores and top-k of T query rows of one sequence against its
 * committed keys, in query-row chunks whose fp32 logits stay within
 * budget_bytes (ATOM PR #1709, commit on right-sizing the prefill logits:
 * the width is the batch's actual maximum committed length, known on the
 * host without a device sync, and Q-row budget chunking rebuilds the
 * schedule per chunk because it encodes absolute row ids). Row r sees
 * visible_end[r] tokens. The result does not depend on budget_bytes.
 *
 *   block_table    int32 [ceil(max visible_end / P)] physical pages of the
 *                  sequence
 *   visible_end    int32 [T], device
 *   W              host: logits width, >= every visible_end[r] (the
 *                  right-sized width max_r visible_end[r])
 *   logits_scratch fp32, scratch_bytes >= idx_prefill_scratch_bytes(T, W, budget)
 *   cta_scratch    int32, cta_scratch_ints >= idx_prefill_schedule_ints(...)
 *   index_base     host, >= 0: added to every selected index (padding stays
 *                  -1). 0 gives sequence-local indices (the FP4 path's output
 *                  in ATOM PR #1709); the sequence's first token in the
 *                  batch's flattened key order gives the GLOBAL indices of
 *                  that page's FP8 prefill path. index_base + W < 2^31.
 *   out_idx        int32 [T][k], ascending indices as in idx_topk, plus
 *                  index_base
 * One launch builds every chunk's schedule (each encodes its chunk's absolute
 * rows, in its own part of cta_scratch); the host loop over chunks then
 * enqueues scores and top-k per chunk on `stream` without synchronizing.
 * A row that sees at most k keys selects all of them, so it needs no scores:
 * blocks of rows that all do are not scored, and logits_scratch is workspace
 * whose rows for them are left as they were.
 * Errors: as idx_paged_mqa_logits and idx_topk; IDX_ERR_WORKSPACE when a
 * scratch buffer is too small.
 */
idx_status idx_prefill_chunked_topk(const idx_query *q, const idx_kv_cache *kv,
                                    const int32_t *block_table, const int32_t *visible_end,
                                    int32_t T, int64_t W, int64_t budget_bytes, int32_t k,
                                    int32_t index_base, float *logits_scratch,
                                    int64_t scratch_bytes, int32_t *cta_scratch,
                                    int64_t cta_scratch_ints, int32_t *out_idx, void *stream);

/* Capacity of the fixed device scratch of idx_prefill_chunked_topk_noalloc:
 * fp32 logits bytes and schedule int32 entries, one copy per GPU. */
#define IDX_NOALLOC_LOGITS_BYTES (64ll << 20)
#define IDX_NOALLOC_SCHEDULE_INTS (1ll << 18)

/*
 * idx_prefill_chunked_topk for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same scores and selection, with the two scratch buffers
 * (the chunk's fp32 logits and every chunk's schedule) taken from a fixed
 * array in the library's own device memory instead of from the caller. The
 * array (IDX_NOALLOC_LOGITS_BYTES + 4 * IDX_NOALLOC_SCHEDULE_INTS bytes,
 * 65 MiB) exists once per GPU the library runs on and is held until the
 * process ends; the call makes no allocation. Its address on the current
 * device is looked up on the first call on that device (one
 * hipGetSymbolAddress; make that first call outside graph capture).
 *   Arguments as idx_prefill_chunked_topk without the scratch buffers.
 *   budget_bytes is capped at IDX_NOALLOC_LOGITS_BYTES; the selection does
 *   not depend on the budget, so out_idx is identical to what
 *   idx_prefill_chunked_topk writes for the same inputs.
 * Every call on one GPU uses the same array: calls that overlap on one GPU
 * (other streams, other host threads) race and must be serialized by the
 * caller. Nothing in the array needs to start at zero (every entry is
 * written before it is read), so no call clears it.
 * Errors: those of idx_prefill_chunked_topk; IDX_ERR_WORKSPACE when the
 * chunk plan for T and W under the capped budget needs more than the fixed
 * scratch holds (more than IDX_NOALLOC_SCHEDULE_INTS schedule entries; e.g.
 * more than 1765888 rows at W = 65536), checked on the host before any
 * HIP call.
 */
idx_status idx_prefill_chunked_topk_noalloc(const idx_query *q, const idx_kv_cache *kv,
                                            const int32_t *block_table,
                                            const int32_t *visible_end, int32_t T, int64_t W,
                                            int64_t budget_bytes, int32_t k, int32_t index_base,
                                            int32_t *out_idx, void *stream);

/* Element type of the rows idx_kv_cache_write and idx_quantize_query
 * quantize. */
typedef enum idx_kin_dtype {
    IDX_KIN_F32 = 0,
    IDX_KIN_BF16 = 1
} idx_kin_dtype;

/*
 * Indexer K-cache writer: quantizes N new key rows of 128 values to the
 * cache's storage format and scatters them into their pages, the step that
 * produces what idx_paged_mqa_logits reads (ATOM PR #1709 names the "FP4
 * mqa-logits / scatter kernels" in the commit adding the FP4 indexer flag).
 *   k             device, N rows of 128 fp32 or bf16 (k_dtype), row r at
 *                 element r*k_row_stride (k_row_stride >= 128 and even; k
 *                 aligned to two elements: 8 bytes fp32, 4 bytes bf16)
 *   slot_mapping  device int64 [N]: row r goes to page slot_mapping[r] / P,
 *                 slot slot_mapping[r] % P; a negative entry or a page at or
 *                 past kv->num_pages skips the row (nothing written)
 *   kv            destination cache (dtype FP8 or MXFP4, same strides as for
 *                 the scores); its data and scale buffers ARE WRITTEN
 * Encoding (readings; the pages name the kernels only):
 *   FP8 E4M3FN: one fp32 scale per row, amax/448 in single precision (1 for
 *   an all-zero row); codes = x/scale rounded to the nearest E4M3 value, ties
 *   to the even code, sign kept.
 *   MXFP4 (OCP MX): per 32 elements the E8M0 exponent floor(log2 amax) - 2,
 *   clamped to [-127, 127] (0 for an all-zero block); codes = x*2^-e rounded
 *   to the nearest E2M1 magnitude, ties to the even code, saturating at 6, the
 *   sign bit only on a nonzero code; the even element in the low nibble.
 * Rows mapping to the same slot race (the result is one of them).
 * Errors: IDX_ERR_INVALID (null pointers, N < 0, bad k_dtype or stride, a
 * cache descriptor that fails the checks of idx_paged_mqa_logits),
 * IDX_ERR_UNSUPPORTED (cache dtype other than FP8 / MXFP4). N = 0 is a no-op.
 */
idx_status idx_kv_cache_write(const void *k, int32_t k_dtype, int64_t k_row_stride, int32_t N,
                              const int64_t *slot_mapping, const idx_kv_cache *kv,
                              void *stream);

/*
 * Indexer query quantization with the weight fold: turns R rows of 64 x 128
 * query values into the query operands of idx_paged_mqa_logits, the step the
 * pages call forward_pre's "quant + weights" (ATOM PR #1709, commit on the
 * forward_pre / score_topk_from split: the FP8 path hands the scorer only the
 * quantized q and the weights, the FP4 path also keeps its q scales).
 *   x      device, R rows of 8192 fp32 or bf16 (x_dtype, idx_kin_dtype), head
 *          h of row r at element r*x_row_stride + 128*h; x 16-byte aligned,
 *          x_row_stride >= 8192 and a multiple of 8
 *   w      device fp32 [R][64], the per-head weights before the fold
 *   c      finite constant multiplied into every weight (e.g. a softmax
 *          scale times 64^-0.5); 1 for none
 *   out    descriptor of the destination query (dtype FP8 or MXFP4, 64
 *          heads, 128 dims, the layout idx_paged_mqa_logits reads); out->q,
 *          out->q_scale (when not NULL) and out->weights ARE WRITTEN. out->
 *          weights may equal w (in place).
 * Encoding (readings; the pages name the step only):
 *   FP8 E4M3FN: one scale per row s = amax/448 over its 8192 values in single
 *   precision (1 for an all-zero row); codes = x/s rounded as the K-cache
 *   writer rounds. With out->q_scale NULL the scale is folded into the
 *   weights, weights = (w*s)*c (fp32, in that order; valid because
 *   max(0, s*y) = s*max(0, y) for s > 0), and the scorer is called with
 *   q_scale NULL. With out->q_scale set, it receives s and weights = w*c.
 *   MXFP4: per 32 values the OCP MX exponent and E2M1 codes exactly as the K-
 *   cache writer encodes a key row, scales to out->q_scale [R][64][4]
 *   (required; a per-block scale does not fold into a per-head weight);
 *   weights = w*c.
 * Errors: IDX_ERR_INVALID (null pointers when R > 0, R < 0, bad x_dtype,
 * stride or alignment, c not finite, a destination that fails the query
 * checks of idx_paged_mqa_logits), IDX_ERR_UNSUPPORTED (dtype or shape).
 * R = 0 is a no-op.
 */
idx_status idx_quantize_query(const void *x, int32_t x_dtype, int64_t x_row_stride, int32_t R,
                              const float *w, float c, const idx_query *out, void *stream);

/* Paged cache of bf16 latent rows (512 values) for the sparse attention:
 * token slot s of physical page p at data + p*page_stride_bytes +
 * s*row_stride_bytes. data 16-byte aligned; strides multiples of 16;
 * row_stride_bytes >= 1024; page_stride_bytes >= page_size*row_stride_bytes. */
typedef struct idx_mla_cache {
    int32_t page_size; /* 32, 64 or 256 */
    int32_t reserved;  /* set to 0 */
    int64_t num_pages;
    const void *data;
    int64_t page_stride_bytes;
    int64_t row_stride_bytes;
} idx_mla_cache;

/* Workspace bytes idx_sparse_mla_decode needs for R rows and lists of k. */
size_t idx_sparse_mla_workspace_size(int32_t R, int32_t k);

/*
 * Sparse attention over the indexer's selection (the consumer of the top-k:
 * flashinfer PR #3269 "Add DeepSeek V4 sparse MLA TRTLLM-GEN kernels", a
 * decode over dynamic per-row top-k lengths with 512-dim QK and V; the
 * values are the latent rows themselves). Row r = b*next_n + j:
 *   n_r = min(topk_lens[r], k) entries of indices[r*k ..] (sequence-local
 *   token ids, e.g. idx_topk's output and counts; entries < 0 are skipped),
 *   s_i = scale * (q[r][h] . c[t_i]),  out[r][h] = sum_i softmax(s)_i c[t_i],
 *   lse[r][h] = log sum_i exp(s_i); no listed token: out = 0, lse = -inf.
 *   q     bf16 [R][64][512], 16-byte aligned
 *   kv    the latent cache; c[t] is slot t % P of page block_tables[b][t / P]
 *   out   bf16 [R][64][512] (written), 8-byte aligned
 *   lse   fp32 [R][64] or NULL
 *   ws    at least idx_sparse_mla_workspace_size(R, k) bytes, 16-byte aligned
 * Listed tokens must lie inside the sequence's pages (device contract, not
 * checked); a table entry outside the pool reads a zero row instead of
 * faulting. Arithmetic: bf16 products with fp32 accumulation, probabilities
 * rounded to bf16 for the P.V product, fp32 softmax, bf16 output.
 * Errors: IDX_ERR_INVALID (null pointers, shapes, strides, alignment, scale
 * not finite, B*next_n > 65535), IDX_ERR_WORKSPACE (ws too small).
 */
idx_status idx_sparse_mla_decode(const void *q, const idx_mla_cache *kv,
                                 const int32_t *block_tables, int64_t bt_stride, int32_t B,
                                 int32_t next_n, const int32_t *indices,
                                 const int32_t *topk_lens, int32_t k, float scale, void *out,
                                 float *lse, void *ws, size_t ws_bytes, void *stream);

/*
 * Opt-in device-side check of the decode contracts idx_paged_mqa_logits does
 * not check (they need a sync to check on the host): for each sequence b,
 * 0 <= context_lens[b] <= W (W > 0; W = 0 skips that bound) and
 * context_lens[b] <= bt_stride*page_size, and every block_tables[b][p] of a
 * page p holding a visible token lies in [0, num_pages). Writes int32
 * result[4] on `stream` (device memory, no sync; read it after the stream):
 *   result[0] sequences breaking a length bound, result[1] out-of-pool table
 *   entries of visible pages, result[2] first such sequence, result[3]
 *   sequence of the first such entry (each -1 when there is none).
 * Graph-capturable (the result is cleared by a kernel, not a memset).
 * Errors: IDX_ERR_INVALID (null or misaligned pointers, B outside
 * [0, 16000], bt_stride, page_size, num_pages < 1, W < 0).
 */
idx_status idx_validate_decode(const int32_t *context_lens, int32_t B, const int32_t *block_tables,
                               int64_t bt_stride, int32_t page_size, int64_t num_pages, int64_t W,
                               int32_t *result, void *stream);

/* Human-readable name of a status (static string). */
const char *idx_status_string(idx_status s);

/* Message of the last failed call on this thread ("" if none). */
const char *idx_last_error(void);

/* ABI version of this library (major*10000 + minor*100 + patch). 0.2.0 adds
 * the K-cache writer, the query quantizer, ragged decode, the prefill
 * index_base argument, query flags and decode without a schedule buffer;
 * 0.3.0 adds the sparse attention over the selection and spreads prefill rows
 * evenly over the chunks the budget requires; 0.4.0 adds
 * idx_prefill_chunked_topk_noalloc, limits the decode width to 2^22 and
 * sizes prefill schedules for two-row segments (idx_prefill_schedule_ints). */
int32_t idx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* IDX_H_ */
