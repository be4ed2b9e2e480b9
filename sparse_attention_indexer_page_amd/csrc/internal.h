// Internal launch interface between the C-ABI layer (idx_api.hip) and the
// gfx950 kernels. Not installed; the public interface is include/idx.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "idx.h"

namespace idx {

constexpr int kHeads = 64;   // indexer heads the MFMA tiling is built for
constexpr int kHeadDim = 128; // one 16x16x128 MFMA covers a whole head
constexpr int kTile = 16;    // tokens per MFMA column tile
constexpr int kInlineSplitMaxSegs = 1024; // decode without a schedule buffer: B at most this
constexpr int kMaxSegs = 16000;      // schedule segments the builder scans in LDS (64000 B)
constexpr int kTopkMaxW = 65536;     // in-register top-k row capacity
// Longest segment the work split counts blocks for: every length is clamped
// to this before its blocks are counted, so kMaxSegs segments of 32-token
// blocks sum to less than 2^31 units and no split arithmetic overflows, even
// for lengths that break the device contract (len <= W <= kMaxSegLen).
constexpr int32_t kMaxSegLen = 1 << 22;
__host__ __device__ inline int32_t clamp_seg_len(int32_t v) {
  return v < 0 ? 0 : (v > kMaxSegLen ? kMaxSegLen : v);
}
constexpr int kPrefillRowsPerSeg = 15; // query rows sharing one K stream in prefill
// Work-split cost of entering a segment, in key blocks. Entering a prefill
// row block, each compute wave reloads its query row with a full wait
// (per-group timestamps of seven-row blocks: the groups whose ranges held
// many short segments finished last at a cost of 1; 3 took 1.5-2% off the
// longer chunk of the 16384-row prefill).
constexpr int kPrefillEntryCost = 3;
// A decode sequence's query rows are next_n x 8 KB of FP8, the bytes of
// next_n x 64 key rows, loaded with a full wait when the wave enters the
// sequence: its entry is charged that many key rows, in blocks (1 for one
// row on 64-token blocks, 4 for two rows on 32-token blocks). Measured on the
// MTP length mix, where a quarter of the sequences are empty or shorter than
// one page: scoring 45.6 / 43.8 / 43.5 / 42.6 us at a cost of 0 / 1 / 2 / 4;
// the batched decode 30.9 / 30.7 us at 0 / 1 and 31.8 us at 4.
__host__ __device__ inline int decode_entry_cost(int next_n, int block_tokens) {
  return (next_n * 64 + block_tokens - 1) / block_tokens;
}

// Tokens per schedule block: a block never straddles two pages.
inline int block_tokens(int page_size) { return page_size < 64 ? page_size : 64; }

// LDS of one decode scoring work group: a ring of four slots, each a block's
// key rows (128 B FP8, 64 B MXFP4 per token) and 256 B of scale words, plus
// the 1 KB output stage of each query row. The kernel checks its own size
// against this; the work-group count the library recommends follows from it.
__host__ __device__ constexpr int decode_ring_slots() { return 4; }
__host__ __device__ constexpr int decode_lds_bytes(bool fp8, int block_tokens, int next_n) {
  return decode_ring_slots() * ((fp8 ? 128 : 64) * block_tokens + 256) + next_n * 1024;
}
constexpr int kLdsBytesPerCu = 160 * 1024;

enum SegMode : int {
  kSegDecode = 0,  // segment = sequence; length = context_lens[s]
  kSegPrefill = 1, // segment = kPrefillRowsPerSeg consecutive query rows;
                   // length = max visible_end over those rows, or 0 when that
                   // is at most skip_len (every row then selects all its keys)
};

struct ScheduleArgs {
  const int32_t *lens; // decode: context_lens [nseg]; prefill: visible_end [T]
  int32_t nseg;
  int32_t mode;       // SegMode
  int32_t row0;       // prefill: first query row of the chunk
  int32_t row_end;    // prefill: one past the last query row of the chunk
  int32_t block_tokens;
  int32_t entry_cost; // cost of entering a non-empty segment, in blocks
  int32_t skip_len;   // prefill: a segment of length <= skip_len has no blocks (0: none skipped)
  int32_t n_ctas;
  int32_t *cta_info; // [n_ctas + 1][2]
  // prefill: work group g builds the schedule of rows [row0 + g*chunk_rows,
  // min(row0 + (g+1)*chunk_rows, row_end)) into cta_info + g*chunk_ints
  // (n_chunks work groups; decode: 1)
  int32_t n_chunks;
  int32_t chunk_rows;
  int64_t chunk_ints;
};

struct LogitsArgs {
  // query side
  const uint8_t *q;       // FP8 [R][64][128] / MXFP4 [R][64][64]
  const uint8_t *q_scale; // FP8 fp32 [R] or null / MXFP4 e8m0 [R][64][4]
  const float *weights;   // [R][64]
  // K cache
  const uint8_t *kdata;
  int64_t page_stride;
  int64_t row_stride;
  const uint8_t *kscale;
  int64_t scale_page_stride;
  int64_t scale_row_stride;
  int64_t num_pages;
  int32_t page_size;
  int32_t block_tokens;
  // addressing
  const int32_t *block_tables; // decode [B][bt_stride]; prefill one row
  int64_t bt_stride;           // 0 in prefill (all segments share one table)
  int64_t bt_cols;             // readable entries per block-table row
  const int32_t *lens;         // decode context_lens [B]; prefill visible_end [T]
  int32_t nseg;                // decode B; prefill segments of the chunk
  int32_t next_n;              // decode rows per sequence (the most, with row_offsets)
  const int32_t *row_offsets;  // decode varlen: sequence s owns rows [off[s], off[s+1]); or null
  int32_t row_cap;             // decode varlen: rows the query and logits buffers hold
  int32_t row0;                // prefill: first row of the chunk
  int32_t row_end;             // prefill: end row of the chunk
  int32_t skip_len;            // prefill: a row block whose rows all see at most this many
                               // keys is not scored (its top-k is every visible key)
  const int32_t *cta_info;
  int32_t n_ctas;
  int32_t lead_ctas; // decode without cta_info: when the launch holds two work groups per SIMD,
                     // the first lead_ctas (dispatched first, one per SIMD) take 4/3 of a
                     // share each; 0: equal shares
  // output
  float *logits; // decode [B*next_n][W]; prefill [row_end-row0][W]
  int64_t W;
};

struct TopkArgs {
  const float *logits;
  int64_t W;
  const int32_t *lens; // decode: context_lens [B]; rows: per-row lengths [R]
  int32_t next_n;      // rows per length entry (1 for per-row lengths)
  int32_t R;           // rows
  int32_t k;
  int32_t *out_idx;   // [R][k]
  int32_t *out_count; // [R] or null
  int32_t index_base;  // added to every selected index (0: sequence-local)
};

struct KvWriteArgs {
  const void *k;       // [N][128] fp32 or bf16 rows
  int32_t k_bf16;      // 1: bf16 input, 0: fp32
  int64_t k_row_stride; // elements between rows
  int32_t N;
  const int64_t *slot_mapping; // [N]: page * P + slot, < 0 skips the row
  int32_t dtype;       // IDX_FP8_E4M3 / IDX_MXFP4 (cache format)
  uint8_t *data;
  int64_t page_stride;
  int64_t row_stride;
  uint8_t *scale;
  int64_t scale_page_stride;
  int64_t scale_row_stride;
  int64_t num_pages;
  int32_t page_shift; // log2 of the page size
};

struct QQuantArgs {
  const void *x;        // [R][64][128] fp32 or bf16
  int32_t x_bf16;
  int64_t x_row_stride; // elements between rows
  int32_t R;
  int32_t dtype;        // IDX_FP8_E4M3 / IDX_MXFP4
  const float *w;       // [R][64]
  float c;              // constant folded into the weights
  uint8_t *q;           // codes: FP8 [R][8192] / MXFP4 [R][4096]
  uint8_t *q_scale;     // FP8: fp32 [R] or null (folded); MXFP4: E8M0 [R][256]
  float *w_out;         // [R][64]
};

// Listed entries one sparse-attention work group takes (its table of row
// addresses lives in LDS).
constexpr int kMlaMaxChunk = 512;

struct MlaArgs {
  const uint16_t *q;  // bf16 [R][64][512]
  const uint8_t *kv;  // bf16 latent rows of 512
  int64_t page_stride;
  int64_t row_stride;
  int32_t page_size;
  int32_t page_shift;
  int64_t num_pages;
  const int32_t *block_tables;
  int64_t bt_stride;
  int32_t next_n;
  int32_t R;
  const int32_t *indices; // [R][k]
  int32_t k;
  const int32_t *topk_lens; // [R]
  float scale;
  int32_t nsplit; // chunks per row
  int32_t chunk;  // listed entries per chunk, a multiple of 16, <= kMlaMaxChunk
  float *ws_o;    // [R][nsplit][64][512]
  float *ws_ml;   // [R][nsplit][64][2]
  uint16_t *out;  // bf16 [R][64][512]
  float *lse;     // [R][64] or null
};

struct ValidateArgs {
  const int32_t *lens;         // [B]
  int32_t B;
  const int32_t *block_tables; // [B][bt_stride]
  int64_t bt_stride;
  int32_t bt_cols;             // entries per row the scores may read
  int32_t page_size;
  int64_t num_pages;
  int64_t W;                   // logits width, or 0: not checked
  int32_t *result;             // [4]
};

hipError_t launch_schedule(const ScheduleArgs &a, hipStream_t s);
hipError_t launch_validate_decode(const ValidateArgs &a, hipStream_t s);
hipError_t launch_sparse_mla(const MlaArgs &a, hipStream_t s);
hipError_t launch_q_quant(const QQuantArgs &a, hipStream_t s);
hipError_t launch_fill_tail(const int32_t *lens, const int32_t *row_offsets, int32_t B, int32_t n,
                            int64_t W, float *logits, hipStream_t s);
hipError_t launch_varlen_windows(const int32_t *lens, const int32_t *row_offsets, int32_t B,
                                 int32_t max_q, int32_t *visible_end, hipStream_t s);
hipError_t launch_kv_write(const KvWriteArgs &a, hipStream_t s);
hipError_t launch_logits_fp8_decode(const LogitsArgs &a, hipStream_t s);
hipError_t launch_logits_mxfp4_decode(const LogitsArgs &a, hipStream_t s);
hipError_t launch_logits_fp8_prefill(const LogitsArgs &a, hipStream_t s);
hipError_t launch_logits_mxfp4_prefill(const LogitsArgs &a, hipStream_t s);
hipError_t launch_topk(const TopkArgs &a, hipStream_t s);

} // namespace idx
