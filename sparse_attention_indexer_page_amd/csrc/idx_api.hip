// C ABI of the indexer library: host-side validation and kernel dispatch.
// Every check here runs before any HIP call, so a rejected call leaves the
// device untouched; nothing here allocates, frees or synchronizes.
#include <atomic>
#include <cmath>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "internal.h"

namespace {

thread_local char g_last_error[512] = "";

idx_status fail(idx_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

idx_status ok() {
  g_last_error[0] = '\0';
  return IDX_OK;
}

idx_status hip_fail(hipError_t e, const char *what) {
  return fail(IDX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_page_size(int32_t p) { return p == 32 || p == 64 || p == 256; }

constexpr int32_t kMaxCtas = 1 << 20;

idx_status check_query(const idx_query *q) {
  if (!q) return fail(IDX_ERR_INVALID, "query descriptor is null");
  if (q->dtype != IDX_FP8_E4M3 && q->dtype != IDX_MXFP4)
    return fail(IDX_ERR_UNSUPPORTED, "query dtype %d is not FP8_E4M3 (1) or MXFP4 (2)", q->dtype);
  if (q->num_heads != idx::kHeads)
    return fail(IDX_ERR_UNSUPPORTED, "num_heads %d unsupported (64 only)", q->num_heads);
  if (q->head_dim != idx::kHeadDim)
    return fail(IDX_ERR_UNSUPPORTED, "head_dim %d unsupported (128 only)", q->head_dim);
  if (q->flags & ~IDX_QUERY_FILL_NEG_INF)
    return fail(IDX_ERR_INVALID, "query flags 0x%x has unknown bits", (unsigned)q->flags);
  if (!q->q || !q->weights) return fail(IDX_ERR_INVALID, "q or weights pointer is null");
  if (!aligned(q->q, 16)) return fail(IDX_ERR_INVALID, "q must be 16-byte aligned");
  if (!aligned(q->weights, 16)) return fail(IDX_ERR_INVALID, "weights must be 16-byte aligned");
  if (q->dtype == IDX_MXFP4 && !q->q_scale)
    return fail(IDX_ERR_INVALID, "MXFP4 queries need their E8M0 scales (q_scale)");
  if (q->dtype == IDX_FP8_E4M3 && q->q_scale && !aligned(q->q_scale, 4))
    return fail(IDX_ERR_INVALID, "FP8 q_scale must be 4-byte aligned");
  return IDX_OK;
}

idx_status check_cache(const idx_kv_cache *kv, int32_t dtype) {
  if (!kv) return fail(IDX_ERR_INVALID, "kv cache descriptor is null");
  if (kv->dtype != dtype)
    return fail(IDX_ERR_UNSUPPORTED, "kv dtype %d differs from query dtype %d", kv->dtype, dtype);
  if (!valid_page_size(kv->page_size))
    return fail(IDX_ERR_INVALID, "page_size %d not in {32, 64, 256}", kv->page_size);
  if (!kv->data || !kv->scale) return fail(IDX_ERR_INVALID, "kv data or scale pointer is null");
  if (kv->num_pages < 1) return fail(IDX_ERR_INVALID, "num_pages must be >= 1");
  const int64_t row_bytes = dtype == IDX_FP8_E4M3 ? idx::kHeadDim : idx::kHeadDim / 2;
  if (!aligned(kv->data, 16) || kv->row_stride_bytes % 16 || kv->page_stride_bytes % 16)
    return fail(IDX_ERR_INVALID, "kv data pointer and strides must be multiples of 16 bytes");
  if (kv->row_stride_bytes < row_bytes)
    return fail(IDX_ERR_INVALID, "row_stride_bytes %lld below the %lld-byte row",
                (long long)kv->row_stride_bytes, (long long)row_bytes);
  if (kv->page_stride_bytes < (int64_t)(kv->page_size - 1) * kv->row_stride_bytes + row_bytes)
    return fail(IDX_ERR_INVALID, "page_stride_bytes too small for page_size rows");
  if ((int64_t)kv->page_size * kv->row_stride_bytes >= (1ll << 31))
    return fail(IDX_ERR_INVALID, "page extent must stay below 2 GiB");
  if (!aligned(kv->scale, 4) || kv->scale_row_stride_bytes % 4 || kv->scale_page_stride_bytes % 4)
    return fail(IDX_ERR_INVALID, "kv scale pointer and strides must be multiples of 4 bytes");
  if (kv->scale_row_stride_bytes < 4)
    return fail(IDX_ERR_INVALID, "scale_row_stride_bytes must be >= 4");
  if ((int64_t)kv->page_size * kv->scale_row_stride_bytes >= (1ll << 31))
    return fail(IDX_ERR_INVALID, "scale page extent must stay below 2 GiB");
  return IDX_OK;
}

// Compute units of the current device, looked up once per device (0 when
// none is present).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

idx::LogitsArgs logits_args(const idx_query *q, const idx_kv_cache *kv) {
  idx::LogitsArgs a;
  memset(&a, 0, sizeof a);
  a.q = static_cast<const uint8_t *>(q->q);
  a.q_scale = static_cast<const uint8_t *>(q->q_scale);
  a.weights = q->weights;
  a.kdata = static_cast<const uint8_t *>(kv->data);
  a.page_stride = kv->page_stride_bytes;
  a.row_stride = kv->row_stride_bytes;
  a.kscale = static_cast<const uint8_t *>(kv->scale);
  a.scale_page_stride = kv->scale_page_stride_bytes;
  a.scale_row_stride = kv->scale_row_stride_bytes;
  a.num_pages = kv->num_pages;
  a.page_size = kv->page_size;
  a.block_tokens = idx::block_tokens(kv->page_size);
  return a;
}

int64_t prefill_rows_per_chunk(int64_t W, int64_t budget) {
  int64_t rows = budget / (4 * W);
  return rows < 1 ? 1 : rows;
}

// Rows of one prefill chunk actually used: the budget rule, capped so the
// schedule builder's segment scan fits in LDS, then spread evenly over the
// chunks that rule needs (n = ceil(T / max rows), ceil(T / n) rows each), so
// no chunk is a small remainder that leaves most of the chip idle (the
// result does not depend on the chunking).
int64_t prefill_chunk_rows(int32_t T, int64_t W, int64_t budget) {
  int64_t rows = prefill_rows_per_chunk(W, budget);
  const int64_t cap = (int64_t)idx::kMaxSegs * idx::kPrefillRowsPerSeg;
  if (rows > cap) rows = cap;
  if (rows > T) rows = T;
  if (rows < 1) rows = 1;
  const int64_t n = (T + rows - 1) / rows;
  rows = (T + n - 1) / n; // <= the budget's rows
  return rows < 1 ? 1 : rows;
}

// Work groups of a prefill chunk: one per block of query rows, at most 256
// (one resident 16-wave group per CU of an MI355X; each walks an equal share
// of the chunk's key blocks).
int32_t prefill_ctas(int64_t chunk_rows) {
  int64_t segs = (chunk_rows + idx::kPrefillRowsPerSeg - 1) / idx::kPrefillRowsPerSeg;
  if (segs < 1) segs = 1;
  return (int32_t)(segs < 256 ? segs : 256);
}

// Fixed device scratch of the no-allocation prefill entry: the chunk's fp32
// logits, then the chunks' schedules. One copy per GPU the library runs on,
// held until the process ends. In host code `g_noalloc_scratch` names a
// host-side stand-in, not device memory: every host use goes through the
// device address hipGetSymbolAddress returns for the current device.
constexpr int64_t kNoAllocLogitsBytes = IDX_NOALLOC_LOGITS_BYTES;
constexpr int64_t kNoAllocScheduleInts = IDX_NOALLOC_SCHEDULE_INTS;
__device__ __align__(256) uint8_t g_noalloc_scratch[kNoAllocLogitsBytes + 4 * kNoAllocScheduleInts];

constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
uint8_t *g_noalloc_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up once per device
// (with that device current) and kept.
idx_status noalloc_scratch(uint8_t **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(IDX_ERR_UNSUPPORTED, "device %d beyond the %d devices the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (g_noalloc_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_noalloc_scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_noalloc_ptr[dev] = static_cast<uint8_t *>(p);
  }
  *out = g_noalloc_ptr[dev];
  return IDX_OK;
}

} // namespace

extern "C" {

int32_t idx_version(void) { return 400; }

const char *idx_status_string(idx_status s) {
  switch (s) {
  case IDX_OK: return "IDX_OK";
  case IDX_ERR_INVALID: return "IDX_ERR_INVALID";
  case IDX_ERR_UNSUPPORTED: return "IDX_ERR_UNSUPPORTED";
  case IDX_ERR_WORKSPACE: return "IDX_ERR_WORKSPACE";
  case IDX_ERR_HIP: return "IDX_ERR_HIP";
  }
  return "IDX_ERR_UNKNOWN";
}

const char *idx_last_error(void) { return g_last_error; }

int64_t idx_schedule_ints(int32_t n_ctas) { return n_ctas < 1 ? 0 : 2 * ((int64_t)n_ctas + 1); }

int32_t idx_recommended_ctas(int32_t rows) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  int64_t n = (int64_t)cus * 8;
  if (rows > n) n = rows;
  return (int32_t)(n < kMaxCtas ? n : kMaxCtas);
}

idx_status idx_validate_decode(const int32_t *context_lens, int32_t B, const int32_t *block_tables,
                               int64_t bt_stride, int32_t page_size, int64_t num_pages, int64_t W,
                               int32_t *result, void *stream) {
  if (!context_lens || !block_tables || !result)
    return fail(IDX_ERR_INVALID, "null context_lens, block_tables or result");
  if (B < 0 || B > idx::kMaxSegs) return fail(IDX_ERR_INVALID, "B = %d outside [0, %d]", B, idx::kMaxSegs);
  if (bt_stride < 1 || bt_stride > (1 << 30))
    return fail(IDX_ERR_INVALID, "bt_stride %lld outside [1, 2^30]", (long long)bt_stride);
  if (!valid_page_size(page_size))
    return fail(IDX_ERR_INVALID, "page_size %d not in {32, 64, 256}", page_size);
  if (num_pages < 1 || W < 0) return fail(IDX_ERR_INVALID, "num_pages must be >= 1 and W >= 0");
  if (!aligned(result, 4) || !aligned(context_lens, 4) || !aligned(block_tables, 4))
    return fail(IDX_ERR_INVALID, "context_lens, block_tables and result must be 4-byte aligned");
  idx::ValidateArgs a;
  a.lens = context_lens;
  a.B = B;
  a.block_tables = block_tables;
  a.bt_stride = bt_stride;
  a.bt_cols = (int32_t)bt_stride; // the decode scores read up to bt_stride entries per row
  a.page_size = page_size;
  a.num_pages = num_pages;
  a.W = W;
  a.result = result;
  hipError_t e = idx::launch_validate_decode(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "validation launch");
  return ok();
}

int32_t idx_recommended_decode_ctas(int32_t rows, int32_t dtype, int32_t page_size,
                                    int32_t next_n) {
  if ((dtype != IDX_FP8_E4M3 && dtype != IDX_MXFP4) || !valid_page_size(page_size) ||
      next_n < 1 || next_n > 4)
    return 0;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  // batched decode, FP8, 64-row pages: 1024 work groups 29.8 us, 768: 30.7,
  // 1536: 35.6, 2048: 34.7 (four 8.4 KB ring slots per group: four groups
  // per CU); MTP (32-row pages, two rows) and MXFP4 (4.3 KB slots, eight
  // groups per CU): 2048 beat 1024 by 10% and 7%. Two groups per SIMD where
  // the LDS holds eight groups, else one: every group is resident at once.
  const int lds = idx::decode_lds_bytes(dtype == IDX_FP8_E4M3, idx::block_tokens(page_size), next_n);
  const bool big_blocks = dtype == IDX_FP8_E4M3 && idx::block_tokens(page_size) == 64 && next_n == 1;
  const int per_cu = !big_blocks && 8 * lds <= idx::kLdsBytesPerCu ? 8 : 4;
  int64_t n = (int64_t)cus * per_cu;
  if (rows > n) n = rows;
  return (int32_t)(n < kMaxCtas ? n : kMaxCtas);
}

idx_status idx_build_schedule(const int32_t *context_lens, int32_t B, int32_t next_n,
                              int32_t page_size, int32_t n_ctas, int32_t *cta_info,
                              void *stream) {
  if (!context_lens || !cta_info) return fail(IDX_ERR_INVALID, "null context_lens or cta_info");
  if (B < 1 || B > idx::kMaxSegs)
    return fail(IDX_ERR_INVALID, "B = %d outside [1, %d]", B, idx::kMaxSegs);
  if (next_n < 1 || next_n > 4) return fail(IDX_ERR_INVALID, "next_n = %d outside [1, 4]", next_n);
  if (!valid_page_size(page_size))
    return fail(IDX_ERR_INVALID, "page_size %d not in {32, 64, 256}", page_size);
  if (n_ctas < 1 || n_ctas > kMaxCtas)
    return fail(IDX_ERR_INVALID, "n_ctas = %d outside [1, %d]", n_ctas, kMaxCtas);
  idx::ScheduleArgs a;
  a.lens = context_lens;
  a.nseg = B;
  a.mode = idx::kSegDecode;
  a.row0 = 0;
  a.row_end = 0;
  a.block_tokens = idx::block_tokens(page_size);
  a.entry_cost = idx::decode_entry_cost(next_n, a.block_tokens);
  a.skip_len = 0; // decode scores are the call's output: every sequence is scored
  a.n_ctas = n_ctas;
  a.cta_info = cta_info;
  a.n_chunks = 1;
  a.chunk_rows = 0;
  a.chunk_ints = 0;
  hipError_t e = idx::launch_schedule(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "schedule launch");
  return ok();
}

namespace {

idx_status decode_logits(const idx_query *q, const idx_kv_cache *kv, const int32_t *block_tables,
                         int64_t bt_stride, const int32_t *context_lens,
                         const int32_t *row_offsets, int32_t B, int32_t next_n,
                         const int32_t *cta_info, int32_t n_ctas, float *logits, int64_t W,
                         void *stream) {
  idx_status st = check_query(q);
  if (st != IDX_OK) return st;
  if ((st = check_cache(kv, q->dtype)) != IDX_OK) return st;
  if (!block_tables || !context_lens || !logits)
    return fail(IDX_ERR_INVALID, "null block_tables, context_lens or logits");
  if (B < 1 || B > idx::kMaxSegs)
    return fail(IDX_ERR_INVALID, "B = %d outside [1, %d]", B, idx::kMaxSegs);
  if (!cta_info && B > idx::kInlineSplitMaxSegs)
    return fail(IDX_ERR_INVALID, "without cta_info B = %d must be <= %d", B,
                idx::kInlineSplitMaxSegs);
  if (next_n < 1 || next_n > 4) return fail(IDX_ERR_INVALID, "next_n = %d outside [1, 4]", next_n);
  if (bt_stride < 1) return fail(IDX_ERR_INVALID, "bt_stride must be >= 1");
  if (n_ctas < 1 || n_ctas > kMaxCtas)
    return fail(IDX_ERR_INVALID, "n_ctas = %d outside [1, %d]", n_ctas, kMaxCtas);
  if (W < 1 || W > idx::kMaxSegLen)
    return fail(IDX_ERR_INVALID, "W = %lld outside [1, 2^22]", (long long)W);
  idx::LogitsArgs a = logits_args(q, kv);
  a.block_tables = block_tables;
  a.bt_stride = bt_stride;
  a.bt_cols = bt_stride;
  a.lens = context_lens;
  a.nseg = B;
  a.next_n = next_n;
  a.row_offsets = row_offsets;
  a.row_cap = B * next_n;
  a.cta_info = cta_info;
  a.n_ctas = n_ctas;
  const int cus = device_cus();
  a.lead_ctas = !cta_info && cus > 0 && cus <= 1024 && n_ctas == 8 * cus ? 4 * cus : 0;
  a.logits = logits;
  a.W = W;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = q->dtype == IDX_FP8_E4M3 ? idx::launch_logits_fp8_decode(a, s)
                                          : idx::launch_logits_mxfp4_decode(a, s);
  if (e != hipSuccess) return hip_fail(e, "logits launch");
  if (q->flags & IDX_QUERY_FILL_NEG_INF) {
    e = idx::launch_fill_tail(context_lens, row_offsets, B, next_n, W, logits, s);
    if (e != hipSuccess) return hip_fail(e, "logits tail launch");
  }
  return ok();
}

} // namespace

idx_status idx_paged_mqa_logits(const idx_query *q, const idx_kv_cache *kv,
                                const int32_t *block_tables, int64_t bt_stride,
                                const int32_t *context_lens, int32_t B, int32_t next_n,
                                const int32_t *cta_info, int32_t n_ctas, float *logits,
                                int64_t W, void *stream) {
  return decode_logits(q, kv, block_tables, bt_stride, context_lens, nullptr, B, next_n,
                       cta_info, n_ctas, logits, W, stream);
}

idx_status idx_paged_mqa_logits_varlen(const idx_query *q, const idx_kv_cache *kv,
                                       const int32_t *block_tables, int64_t bt_stride,
                                       const int32_t *context_lens, const int32_t *row_offsets,
                                       int32_t B, int32_t max_q, const int32_t *cta_info,
                                       int32_t n_ctas, float *logits, int64_t W, void *stream) {
  if (!row_offsets) return fail(IDX_ERR_INVALID, "row_offsets is null");
  if (!aligned(row_offsets, 4)) return fail(IDX_ERR_INVALID, "row_offsets misaligned");
  return decode_logits(q, kv, block_tables, bt_stride, context_lens, row_offsets, B, max_q,
                       cta_info, n_ctas, logits, W, stream);
}

idx_status idx_varlen_windows(const int32_t *context_lens, const int32_t *row_offsets, int32_t B,
                              int32_t max_q, int32_t *visible_end, void *stream) {
  if (!context_lens || !row_offsets || !visible_end)
    return fail(IDX_ERR_INVALID, "null context_lens, row_offsets or visible_end");
  if (B < 1 || B > idx::kMaxSegs)
    return fail(IDX_ERR_INVALID, "B = %d outside [1, %d]", B, idx::kMaxSegs);
  if (max_q < 1 || max_q > 4) return fail(IDX_ERR_INVALID, "max_q = %d outside [1, 4]", max_q);
  if (!aligned(context_lens, 4) || !aligned(row_offsets, 4) || !aligned(visible_end, 4))
    return fail(IDX_ERR_INVALID, "misaligned int32 arrays");
  hipError_t e = idx::launch_varlen_windows(context_lens, row_offsets, B, max_q, visible_end,
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "windows launch");
  return ok();
}

size_t idx_topk_workspace_size(int32_t rows, int64_t W, int32_t k) {
  (void)rows;
  (void)W;
  (void)k;
  return 0;
}

idx_status idx_topk(const float *logits, int64_t W, const int32_t *context_lens, int32_t B,
                    int32_t next_n, int32_t k, int32_t *out_idx, int32_t *out_count, void *ws,
                    size_t ws_bytes, void *stream) {
  (void)ws;
  if (!logits || !context_lens || !out_idx)
    return fail(IDX_ERR_INVALID, "null logits, context_lens or out_idx");
  if (B < 1) return fail(IDX_ERR_INVALID, "B must be >= 1");
  if (next_n < 1 || next_n > 4) return fail(IDX_ERR_INVALID, "next_n = %d outside [1, 4]", next_n);
  if (W < 1) return fail(IDX_ERR_INVALID, "W must be >= 1");
  if (k < 1) return fail(IDX_ERR_INVALID, "k = %d must be >= 1", k);
  if (W > idx::kTopkMaxW)
    return fail(IDX_ERR_UNSUPPORTED, "W = %lld above the %d-wide in-register top-k", (long long)W,
                idx::kTopkMaxW);
  if ((int64_t)B * next_n > (1ll << 31) - 1) return fail(IDX_ERR_INVALID, "too many rows");
  if (ws_bytes < idx_topk_workspace_size(B * next_n, W, k))
    return fail(IDX_ERR_WORKSPACE, "top-k workspace too small");
  idx::TopkArgs a;
  a.logits = logits;
  a.W = W;
  a.lens = context_lens;
  a.next_n = next_n;
  a.R = B * next_n;
  a.k = k;
  a.out_idx = out_idx;
  a.out_count = out_count;
  a.index_base = 0;
  hipError_t e = idx::launch_topk(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  return ok();
}

idx_status idx_kv_cache_write(const void *k, int32_t k_dtype, int64_t k_row_stride, int32_t N,
                              const int64_t *slot_mapping, const idx_kv_cache *kv,
                              void *stream) {
  if (!kv) return fail(IDX_ERR_INVALID, "kv cache descriptor is null");
  if (kv->dtype != IDX_FP8_E4M3 && kv->dtype != IDX_MXFP4)
    return fail(IDX_ERR_UNSUPPORTED, "cache dtype %d is neither FP8 nor MXFP4", kv->dtype);
  idx_status st;
  if ((st = check_cache(kv, kv->dtype)) != IDX_OK) return st;
  if (N < 0) return fail(IDX_ERR_INVALID, "N = %d must be >= 0", N);
  if (k_dtype != IDX_KIN_F32 && k_dtype != IDX_KIN_BF16)
    return fail(IDX_ERR_INVALID, "k_dtype %d is neither fp32 nor bf16", k_dtype);
  if (k_row_stride < idx::kHeadDim)
    return fail(IDX_ERR_INVALID, "k_row_stride %lld below the %d-value row",
                (long long)k_row_stride, idx::kHeadDim);
  if (N == 0) return ok();
  if (!k || !slot_mapping) return fail(IDX_ERR_INVALID, "null k or slot_mapping");
  // rows are read two values at a time: 8-byte (fp32) / 4-byte (bf16) alignment
  const size_t pair = k_dtype == IDX_KIN_F32 ? 8 : 4;
  if (!aligned(k, pair) || k_row_stride % 2 || !aligned(slot_mapping, 8))
    return fail(IDX_ERR_INVALID, "k (pairs of values), k_row_stride (even) or slot_mapping "
                                 "misaligned");
  idx::KvWriteArgs a;
  a.k = k;
  a.k_bf16 = k_dtype == IDX_KIN_BF16;
  a.k_row_stride = k_row_stride;
  a.N = N;
  a.slot_mapping = slot_mapping;
  a.dtype = kv->dtype;
  a.data = static_cast<uint8_t *>(const_cast<void *>(kv->data));
  a.page_stride = kv->page_stride_bytes;
  a.row_stride = kv->row_stride_bytes;
  a.scale = static_cast<uint8_t *>(const_cast<void *>(kv->scale));
  a.scale_page_stride = kv->scale_page_stride_bytes;
  a.scale_row_stride = kv->scale_row_stride_bytes;
  a.num_pages = kv->num_pages;
  a.page_shift = kv->page_size == 32 ? 5 : (kv->page_size == 64 ? 6 : 8);
  hipError_t e = idx::launch_kv_write(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kv write launch");
  return ok();
}

idx_status idx_quantize_query(const void *x, int32_t x_dtype, int64_t x_row_stride, int32_t R,
                              const float *w, float c, const idx_query *out, void *stream) {
  if (!out) return fail(IDX_ERR_INVALID, "query descriptor is null");
  if (out->dtype != IDX_FP8_E4M3 && out->dtype != IDX_MXFP4)
    return fail(IDX_ERR_UNSUPPORTED, "query dtype %d is not FP8_E4M3 (1) or MXFP4 (2)",
                out->dtype);
  if (out->num_heads != idx::kHeads || out->head_dim != idx::kHeadDim)
    return fail(IDX_ERR_UNSUPPORTED, "query shape %d x %d unsupported (64 x 128 only)",
                out->num_heads, out->head_dim);
  if (R < 0) return fail(IDX_ERR_INVALID, "R = %d must be >= 0", R);
  if (x_dtype != IDX_KIN_F32 && x_dtype != IDX_KIN_BF16)
    return fail(IDX_ERR_INVALID, "x_dtype %d is neither fp32 nor bf16", x_dtype);
  if (x_row_stride < (int64_t)idx::kHeads * idx::kHeadDim)
    return fail(IDX_ERR_INVALID, "x_row_stride %lld below the %d-value row",
                (long long)x_row_stride, idx::kHeads * idx::kHeadDim);
  if (!std::isfinite(c)) return fail(IDX_ERR_INVALID, "weight constant is not finite");
  if (R == 0) return ok();
  idx_status st = check_query(out);
  if (st != IDX_OK) return st;
  if (!x || !w) return fail(IDX_ERR_INVALID, "null x or w");
  // eight values per load: 16-byte aligned rows
  if (!aligned(x, 16) || x_row_stride % 8)
    return fail(IDX_ERR_INVALID, "x must be 16-byte aligned and x_row_stride a multiple of 8");
  if (!aligned(w, 4)) return fail(IDX_ERR_INVALID, "w must be 4-byte aligned");
  idx::QQuantArgs a;
  a.x = x;
  a.x_bf16 = x_dtype == IDX_KIN_BF16;
  a.x_row_stride = x_row_stride;
  a.R = R;
  a.dtype = out->dtype;
  a.w = w;
  a.c = c;
  a.q = static_cast<uint8_t *>(const_cast<void *>(out->q));
  a.q_scale = static_cast<uint8_t *>(const_cast<void *>(out->q_scale));
  a.w_out = const_cast<float *>(out->weights);
  hipError_t e = idx::launch_q_quant(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "query quantization launch");
  return ok();
}

namespace {

// Chunks per row of the sparse attention: enough work groups to cover the
// chip (R * nsplit >= 256) with chunks of at least 64 listed entries, and
// never more than kMlaMaxChunk entries per chunk (the kernel's LDS table).
void mla_split(int32_t R, int32_t k, int32_t *nsplit, int32_t *chunk) {
  int32_t ns = R >= 256 ? 1 : (256 + R - 1) / R;
  const int32_t max_ns = (k + 63) / 64;
  ns = ns < max_ns ? ns : max_ns;
  const int32_t min_ns = (k + idx::kMlaMaxChunk - 1) / idx::kMlaMaxChunk;
  ns = ns > min_ns ? ns : min_ns;
  ns = ns < 1 ? 1 : ns;
  int32_t ch = (k + ns - 1) / ns;
  ch = (ch + 15) / 16 * 16; // <= kMlaMaxChunk, a multiple of 16
  *nsplit = (k + ch - 1) / ch;
  *chunk = ch;
}

} // namespace

size_t idx_sparse_mla_workspace_size(int32_t R, int32_t k) {
  if (R < 1 || k < 1) return 0;
  int32_t ns, ch;
  mla_split(R, k, &ns, &ch);
  return (size_t)R * ns * 64 * (512 + 2) * sizeof(float);
}

idx_status idx_sparse_mla_decode(const void *q, const idx_mla_cache *kv,
                                 const int32_t *block_tables, int64_t bt_stride, int32_t B,
                                 int32_t next_n, const int32_t *indices,
                                 const int32_t *topk_lens, int32_t k, float scale, void *out,
                                 float *lse, void *ws, size_t ws_bytes, void *stream) {
  if (!q || !kv || !block_tables || !indices || !topk_lens || !out || !ws)
    return fail(IDX_ERR_INVALID, "null q, kv, block_tables, indices, topk_lens, out or ws");
  if (!valid_page_size(kv->page_size))
    return fail(IDX_ERR_INVALID, "page_size %d not in {32, 64, 256}", kv->page_size);
  if (!kv->data || kv->num_pages < 1) return fail(IDX_ERR_INVALID, "empty latent cache");
  if (!aligned(kv->data, 16) || kv->page_stride_bytes % 16 || kv->row_stride_bytes % 16 ||
      kv->row_stride_bytes < 1024 ||
      kv->page_stride_bytes < (int64_t)kv->page_size * kv->row_stride_bytes)
    return fail(IDX_ERR_INVALID, "latent cache rows must be >= 1024 B, strides multiples of 16");
  if (B < 1) return fail(IDX_ERR_INVALID, "B must be >= 1");
  if (next_n < 1 || next_n > 4) return fail(IDX_ERR_INVALID, "next_n = %d outside [1, 4]", next_n);
  if ((int64_t)B * next_n > 65535) return fail(IDX_ERR_INVALID, "too many rows");
  if (bt_stride < 1) return fail(IDX_ERR_INVALID, "bt_stride must be >= 1");
  if (k < 1) return fail(IDX_ERR_INVALID, "k = %d must be >= 1", k);
  if (!std::isfinite(scale)) return fail(IDX_ERR_INVALID, "scale is not finite");
  if (!aligned(q, 16) || !aligned(out, 8) || !aligned(ws, 16) || (lse && !aligned(lse, 4)))
    return fail(IDX_ERR_INVALID, "q (16 B), out (8 B), ws (16 B) or lse misaligned");
  const int32_t R = B * next_n;
  if (ws_bytes < idx_sparse_mla_workspace_size(R, k))
    return fail(IDX_ERR_WORKSPACE, "workspace %zu B < %zu B", ws_bytes,
                idx_sparse_mla_workspace_size(R, k));
  idx::MlaArgs a;
  a.q = static_cast<const uint16_t *>(q);
  a.kv = static_cast<const uint8_t *>(kv->data);
  a.page_stride = kv->page_stride_bytes;
  a.row_stride = kv->row_stride_bytes;
  a.page_size = kv->page_size;
  a.page_shift = kv->page_size == 32 ? 5 : (kv->page_size == 64 ? 6 : 8);
  a.num_pages = kv->num_pages;
  a.block_tables = block_tables;
  a.bt_stride = bt_stride;
  a.next_n = next_n;
  a.R = R;
  a.indices = indices;
  a.k = k;
  a.topk_lens = topk_lens;
  a.scale = scale;
  mla_split(R, k, &a.nsplit, &a.chunk);
  a.ws_o = static_cast<float *>(ws);
  a.ws_ml = a.ws_o + (size_t)R * a.nsplit * 64 * 512;
  a.out = static_cast<uint16_t *>(out);
  a.lse = lse;
  hipError_t e = idx::launch_sparse_mla(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sparse attention launch");
  return ok();
}

int64_t idx_prefill_rows_per_chunk(int64_t W, int64_t budget_bytes) {
  if (W < 1) return 0;
  return prefill_rows_per_chunk(W, budget_bytes);
}

int64_t idx_prefill_scratch_bytes(int32_t T, int64_t W, int64_t budget_bytes) {
  if (T < 1 || W < 1) return 0;
  return 4 * W * prefill_chunk_rows(T, W, budget_bytes);
}

int64_t idx_prefill_schedule_ints(int32_t T, int64_t W, int64_t budget_bytes) {
  if (T < 1 || W < 1) return 0;
  const int64_t rows = prefill_chunk_rows(T, W, budget_bytes);
  const int64_t chunks = (T + rows - 1) / rows;
  return chunks * idx_schedule_ints(prefill_ctas(rows)); // one schedule per chunk
}

static idx_status prefill_chunked_topk(const idx_query *q, const idx_kv_cache *kv,
                                const int32_t *block_table, const int32_t *visible_end, int32_t T,
                                int64_t W, int64_t budget_bytes, int32_t k, int32_t index_base,
                                float *logits_scratch, int64_t scratch_bytes, int32_t *cta_scratch,
                                int64_t cta_scratch_ints, int32_t *out_idx, void *stream) {
  idx_status st = check_query(q);
  if (st != IDX_OK) return st;
  if ((st = check_cache(kv, q->dtype)) != IDX_OK) return st;
  if (!block_table || !visible_end || !logits_scratch || !cta_scratch || !out_idx)
    return fail(IDX_ERR_INVALID, "null block_table, visible_end, scratch or out_idx");
  if (T < 1) return fail(IDX_ERR_INVALID, "T must be >= 1");
  if (W < 1) return fail(IDX_ERR_INVALID, "W must be >= 1");
  if (W > idx::kTopkMaxW)
    return fail(IDX_ERR_UNSUPPORTED, "W = %lld above the %d-wide in-register top-k", (long long)W,
                idx::kTopkMaxW);
  if (k < 1) return fail(IDX_ERR_INVALID, "k = %d must be >= 1", k);
  if (budget_bytes < 1) return fail(IDX_ERR_INVALID, "budget_bytes must be >= 1");
  if (index_base < 0 || (int64_t)index_base + W > (1ll << 31) - 1)
    return fail(IDX_ERR_INVALID, "index_base %d must be >= 0 with index_base + W < 2^31",
                index_base);
  const int64_t rows = prefill_chunk_rows(T, W, budget_bytes);
  if (scratch_bytes < 4 * W * rows)
    return fail(IDX_ERR_WORKSPACE, "logits scratch %lld B < %lld B", (long long)scratch_bytes,
                (long long)(4 * W * rows));
  const int32_t n_ctas = prefill_ctas(rows);
  const int64_t n_chunks = (T + rows - 1) / rows;
  const int64_t sched_ints = idx_schedule_ints(n_ctas); // per chunk
  if (cta_scratch_ints < n_chunks * sched_ints)
    return fail(IDX_ERR_WORKSPACE, "schedule scratch %lld ints < %lld", (long long)cta_scratch_ints,
                (long long)(n_chunks * sched_ints));
  hipStream_t s = static_cast<hipStream_t>(stream);
  // every chunk's schedule in one launch (work group g builds chunk g's),
  // before the first chunk is scored
  idx::ScheduleArgs sa;
  sa.lens = visible_end;
  sa.nseg = (int32_t)((rows + idx::kPrefillRowsPerSeg - 1) / idx::kPrefillRowsPerSeg);
  sa.mode = idx::kSegPrefill;
  sa.row0 = 0;
  sa.row_end = T;
  sa.block_tokens = idx::block_tokens(kv->page_size);
  sa.entry_cost = idx::kPrefillEntryCost;
  sa.skip_len = k; // rows seeing at most k keys select them all: no scores needed
  sa.n_ctas = n_ctas;
  sa.cta_info = cta_scratch;
  sa.n_chunks = (int32_t)n_chunks;
  sa.chunk_rows = (int32_t)rows;
  sa.chunk_ints = sched_ints;
  if (n_chunks == 1) sa.row_end = (int32_t)rows;
  hipError_t e = idx::launch_schedule(sa, s);
  if (e != hipSuccess) return hip_fail(e, "prefill schedule launch");
  idx::LogitsArgs la = logits_args(q, kv);
  la.block_tables = block_table;
  la.bt_stride = 0;
  la.bt_cols = (W + kv->page_size - 1) / kv->page_size;
  la.lens = visible_end;
  la.next_n = 1;
  la.skip_len = k;
  la.n_ctas = n_ctas;
  la.logits = logits_scratch;
  la.W = W;
  for (int64_t r0 = 0; r0 < T; r0 += rows) {
    const int64_t r1 = r0 + rows < T ? r0 + rows : T;
    const int32_t nseg =
        (int32_t)((r1 - r0 + idx::kPrefillRowsPerSeg - 1) / idx::kPrefillRowsPerSeg);
    la.cta_info = cta_scratch + (r0 / rows) * sched_ints;
    la.nseg = nseg;
    la.row0 = (int32_t)r0;
    la.row_end = (int32_t)r1;
    e = q->dtype == IDX_FP8_E4M3 ? idx::launch_logits_fp8_prefill(la, s)
                                 : idx::launch_logits_mxfp4_prefill(la, s);
    if (e != hipSuccess) return hip_fail(e, "prefill logits launch");
    idx::TopkArgs ta;
    ta.logits = logits_scratch;
    ta.W = W;
    ta.lens = visible_end + r0;
    ta.next_n = 1;
    ta.R = (int32_t)(r1 - r0);
    ta.k = k;
    ta.out_idx = out_idx + r0 * k;
    ta.out_count = nullptr;
    ta.index_base = index_base;
    e = idx::launch_topk(ta, s);
    if (e != hipSuccess) return hip_fail(e, "prefill top-k launch");
  }
  return ok();
}


idx_status idx_prefill_chunked_topk(const idx_query *q, const idx_kv_cache *kv,
                                    const int32_t *block_table, const int32_t *visible_end,
                                    int32_t T, int64_t W, int64_t budget_bytes, int32_t k,
                                    int32_t index_base, float *logits_scratch,
                                    int64_t scratch_bytes, int32_t *cta_scratch,
                                    int64_t cta_scratch_ints, int32_t *out_idx, void *stream) {
  return prefill_chunked_topk(q, kv, block_table, visible_end, T, W, budget_bytes, k, index_base,
                              logits_scratch, scratch_bytes, cta_scratch, cta_scratch_ints,
                              out_idx, stream);
}

idx_status idx_prefill_chunked_topk_noalloc(const idx_query *q, const idx_kv_cache *kv,
                                            const int32_t *block_table,
                                            const int32_t *visible_end, int32_t T, int64_t W,
                                            int64_t budget_bytes, int32_t k, int32_t index_base,
                                            int32_t *out_idx, void *stream) {
  // Size checks first, on the host, before any HIP call.
  if (T < 1) return fail(IDX_ERR_INVALID, "T must be >= 1");
  if (W < 1) return fail(IDX_ERR_INVALID, "W must be >= 1");
  if (W > idx::kTopkMaxW)
    return fail(IDX_ERR_UNSUPPORTED, "W = %lld above the %d-wide in-register top-k", (long long)W,
                idx::kTopkMaxW);
  if (budget_bytes < 1) return fail(IDX_ERR_INVALID, "budget_bytes must be >= 1");
  // The fixed logits scratch is one more cap on the budget; the selection does
  // not depend on the budget, so the result equals idx_prefill_chunked_topk's.
  const int64_t budget = budget_bytes < kNoAllocLogitsBytes ? budget_bytes : kNoAllocLogitsBytes;
  const int64_t need_logits = idx_prefill_scratch_bytes(T, W, budget);
  const int64_t need_ints = idx_prefill_schedule_ints(T, W, budget);
  if (need_logits > kNoAllocLogitsBytes || need_ints > kNoAllocScheduleInts)
    return fail(IDX_ERR_WORKSPACE,
                "T = %d, W = %lld need %lld B of logits and %lld schedule ints; the fixed scratch "
                "holds %lld B and %lld ints",
                T, (long long)W, (long long)need_logits, (long long)need_ints,
                (long long)kNoAllocLogitsBytes, (long long)kNoAllocScheduleInts);
  uint8_t *base = nullptr;
  idx_status st = noalloc_scratch(&base);
  if (st != IDX_OK) return st;
  return prefill_chunked_topk(q, kv, block_table, visible_end, T, W, budget, k, index_base,
                              reinterpret_cast<float *>(base), kNoAllocLogitsBytes,
                              reinterpret_cast<int32_t *>(base + kNoAllocLogitsBytes),
                              kNoAllocScheduleInts, out_idx, stream);
}

} // extern "C"
