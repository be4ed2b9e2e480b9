// Paged MQA scores of the sparse-attention indexer on gfx950.
//
//   logits[r][t] = sum_h w[r][h] * max(0, k_scale[t] * (q[r][h] . k[t]))
//
// (the "mqa-logits" step of ROCm/ATOM PR #1709 "Add fp4 indexer fo dsv4" and
// the "FP8 paged-MQA logits" kernel of vllm-project/DeepGEMM PR #14, which
// name the op; the formula is the stated problem this library implements).
//
// Design (one 64-lane wave per work group; the schedule hands each wave a
// contiguous run of (segment, block) items):
//   * A segment's query rows stay in VGPRs as MFMA A operands: row r, head
//     tile m (heads 16m..16m+15) is one 16x128 operand, 32 bytes per lane.
//   * K is streamed straight from HBM into B operands, one 16-token tile per
//     16x16x128 MFMA; one MFMA therefore yields 16 heads x 16 tokens of full
//     dot products (head_dim 128 = the MFMA's K). FP8 uses the unscaled
//     f8f6f4 form; MXFP4 uses the block-scaled form with the E8M0 scale of
//     each lane's 32-element block as the operand scale.
//   * A block of BK = min(P, 64) tokens lies in one physical page (DeepGEMM
//     PR #14: a 64-row tile would straddle two non-contiguous 32-row pages).
//     Each page gets its own buffer resource whose size is the page's extent,
//     or zero when the block-table entry is not a page of the pool, so a bad
//     page id reads zeros instead of faulting (ATOM PR #1709, commit on the
//     ragged-window refresh: a bounds-check-off buffer load faulted on stale
//     metadata).
//   * Epilogue in registers: ReLU, weight and head sum per lane (16 heads),
//     then a cross-lane sum over the four lane groups done as a reduce-scatter
//     with the gfx950 row-swap instructions; the FP8 per-token K scale and
//     per-row q scale are positive, so they are applied outside the ReLU
//     (relu(s*x) = s*relu(x) for s >= 0), once per token.
//
// Operand lane layout (identical for A and B, which is all a full-length dot
// product needs): lane l serves row/column (l & 15); lane group g = l >> 4
// holds FP8 bytes [16g, 16g+16) and [64+16g, 64+16g+16) of the 128-byte row,
// so each of the two 16-byte loads of a 16-row tile reads 64 contiguous bytes
// per row; for MXFP4 it holds bytes [16g, 16g+16) = elements [32g, 32g+32),
// exactly one E8M0 block. Accumulator layout of the 16x16 f32 MFMA: lane l
// holds column (l & 15), rows 4g..4g+3.
#include "device_common.h"
#include "internal.h"

namespace idx {
namespace {

using namespace dev;


// Query-side registers of one segment.
template <int DT, int NROW> struct QRegs {
  v8i a[NROW][4];    // A operands per row and head tile
  int32_t asc[NROW][4]; // MXFP4: E8M0 scale of the lane's block (byte 0)
  float w[NROW][4][4];  // weight (times FP8 q scale) of the lane's 16 heads
  int32_t E[NROW];      // visible length per row
  int32_t out_row[NROW]; // logits row, or -1 for a padding row
};

// The weights times the rows' FP8 q scales (the scores' per-row factor).
template <int DT, int NROW>
__device__ inline void scale_weights(QRegs<DT, NROW> &Q, const float (&qs)[NROW]) {
#pragma unroll
  for (int i = 0; i < NROW; ++i)
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) Q.w[i][m][j] *= qs[i];
}

// Issues the loads of a segment's query rows: A operands, weights and (FP8)
// the per-row q scales, returned in qs. With WAIT the loads are waited for
// and the weights scaled here; without, the caller does both, so no loaded
// value is consumed before its other loads have gone out.
template <int DT, int NROW, bool WAIT = true>
__device__ inline void load_query(QRegs<DT, NROW> &Q, const LogitsArgs &a, const int32_t *rows,
                                  const int32_t *E, const int32_t *out_rows, float (&qs)[NROW]) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int hl = lane & 15;
#pragma unroll
  for (int i = 0; i < NROW; ++i) {
    Q.E[i] = E[i];
    Q.out_row[i] = out_rows[i];
    const int r = rows[i];
    if (r < 0) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        Q.a[i][m] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        Q.asc[i][m] = 127;
#pragma unroll
        for (int j = 0; j < 4; ++j) Q.w[i][m][j] = 0.f;
      }
      qs[i] = 1.f;
      continue;
    }
    qs[i] = 1.f;
    if (DT == IDX_FP8_E4M3 && a.q_scale != nullptr)
      qs[i] = uniform_load(reinterpret_cast<const float *>(a.q_scale) + r);
    const float *wrow = a.weights + (int64_t)r * kHeads;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int h = 16 * m + hl;
      if (DT == IDX_FP8_E4M3) {
        const v4i *p = reinterpret_cast<const v4i *>(a.q + ((int64_t)r * kHeads + h) * kHeadDim);
        Q.a[i][m] = cat(p[g], p[4 + g]);
      } else {
        const v4i *p = reinterpret_cast<const v4i *>(a.q + ((int64_t)r * kHeads + h) * (kHeadDim / 2));
        const v4i lo = p[g];
        Q.a[i][m] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
        Q.asc[i][m] = a.q_scale[((int64_t)r * kHeads + h) * (kHeadDim / 32) + g];
      }
      const v4f wv = *reinterpret_cast<const v4f *>(wrow + 16 * m + 4 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) Q.w[i][m][j] = wv[j]; // times qs once loaded
    }
  }
  // Wait for the query loads here, once per segment: left outstanding, the
  // compiler's wait for them at their first use would be a full vmcnt(0) in
  // every pass of the block loop, i.e. a wait for the next block's K loads.
  // (The first segment's caller waits itself, after the first block's loads,
  // and then scales the weights: nothing here may consume a loaded value.)
  if (WAIT) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    scale_weights(Q, qs);
  }
}

// Rows, visible lengths and output rows of sequence s of length len (as
// stored, not clamped): its n query rows (next_n, or off[s+1] - off[s] with row offsets), row
// j seeing the first len - (n - 1 - j) keys; the remaining register rows are
// padding (-1). Returns the segment's length. With row offsets the count is
// clamped to [0, next_n] and rows outside [0, row_cap) become padding, so
// malformed offsets can only drop rows, never address outside the buffers.
template <int NROW>
__device__ inline int32_t segment_rows(const LogitsArgs &a, int s, int32_t len, int32_t *rows,
                                       int32_t *E, int32_t *out_rows) {
  int32_t base = s * a.next_n, n = a.next_n;
  if (a.row_offsets != nullptr) {
    base = uniform_load(a.row_offsets + s);
    n = uniform_load(a.row_offsets + s + 1) - base;
    n = n < 0 ? 0 : (n > NROW ? NROW : n);
  }
  int32_t L = 0;
#pragma unroll
  for (int i = 0; i < NROW; ++i) {
    const int r = base + i;
    int32_t e = len - (n - 1 - i);
    e = e > 0 ? e : 0;
    const bool live = i < n && r >= 0 && (a.row_offsets == nullptr || r < a.row_cap);
    rows[i] = live ? r : -1;
    E[i] = live ? e : 0;
    out_rows[i] = live ? r : -1;
    L = live && e > L ? e : L;
  }
  return L;
}

// Length of sequence s (its last row's visible length).
__device__ inline int32_t segment_length(const LogitsArgs &a, int s) {
  return clamp_seg_len(uniform_load(a.lens + s));
}

// Position of a wave in its work group's range of (segment, block) items.
struct Walk {
  int s, blk; // current item
  int se, be; // first item past the range
  int nb;     // blocks of segment s
};

__device__ inline bool in_range(const LogitsArgs &a, const Walk &w) {
  return w.s < a.nseg && (w.s < w.se || (w.s == w.se && w.blk < w.be));
}

// Moves to the first block of the next segment that has blocks.
__device__ inline bool next_segment(const LogitsArgs &a, Walk &w) {
  w.blk = 0;
  while (true) {
    ++w.s;
    if (!in_range(a, w)) return false;
    w.nb = (segment_length(a, w.s) + a.block_tokens - 1) >> __builtin_ctz(a.block_tokens);
    if (w.nb > 0) return true;
  }
}

__device__ inline bool advance(const LogitsArgs &a, Walk &w) {
  if (++w.blk < w.nb) return in_range(a, w);
  return next_segment(a, w);
}

// Inclusive prefix sum over the wave's lanes with DPP moves (no LDS round
// trips): shifts by 1, 2, 4, 8 within each 16-lane row (lanes shifted in from
// outside the row add 0), then row 0's total into rows 1 and 3 and row 1's
// into rows 2 and 3 (row_bcast 15), then the first half's into the second
// (row_bcast 31).
__device__ inline int32_t wave_incl_scan(int32_t v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false); // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false); // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false); // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false); // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false); // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false); // row_bcast:31
  return v;
}

// The range of work group c when no schedule buffer is given: the wave
// computes what the schedule builder would write for entries c and c + 1
// (same costs: ceil(len / BK) blocks per non-empty sequence plus the decode
// entry cost; range c starts at unit floor(c * N / n_ctas) of the N units),
// from all B <= kInlineSplitMaxSegs lengths at once, 64 sequences per lane
// slot.
__device__ inline int32_t own_range(const LogitsArgs &a, int c, Walk &w) {
  constexpr int kChunks = kInlineSplitMaxSegs / 64;
  const int lane = threadIdx.x & 63;
  const int32_t entry = decode_entry_cost(a.next_n, a.block_tokens); // as the schedule builder
  int32_t len[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) // every load first: one round trip
    if (i * 64 < a.nseg) len[i] = 64 * i + lane < a.nseg ? clamp_seg_len(a.lens[64 * i + lane]) : 0;
  int32_t pre[kChunks]; // exclusive prefix cost of sequence 64 i + lane
  int32_t total = 0;
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    if (i * 64 < a.nseg) {
      const int32_t L = len[i]; // clamped to [0, kMaxSegLen]
      const int32_t nb = (L + a.block_tokens - 1) >> __builtin_ctz(a.block_tokens); // 32 or 64
      const int32_t cost = nb > 0 ? nb + entry : 0;
      const int32_t incl = wave_incl_scan(cost);
      pre[i] = total + incl - cost;
      total += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  const int64_t N = total;
  int32_t len0 = 0; // length of the range's first sequence
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    // floor((c + e) N / n_ctas) through one double division: the numerator
    // (< 2^51) and n_ctas (<= 2^20) are exact, and a non-integer quotient
    // (< 2^31) lies at least 1/n_ctas from an integer, far beyond the
    // division's rounding error (< 2^-22), so truncation gives the floor
    const int64_t T = (int64_t)((double)((int64_t)(c + e) * N) / (double)a.n_ctas);
    int32_t seg = a.nseg, blk = 0;
    if (T < N) {
      // the last sequence whose prefix is <= T holds unit T
      int32_t cnt = 0;
#pragma unroll
      for (int i = 0; i < kChunks; ++i)
        if (i * 64 < a.nseg)
          cnt += __popcll(__ballot(64 * i + lane < a.nseg && pre[i] <= T));
      seg = cnt - 1;
      int32_t p = 0;
#pragma unroll
      for (int i = 0; i < kChunks; ++i)
        if (i == (seg >> 6)) {
          p = __builtin_amdgcn_readlane(pre[i], seg & 63);
          if (e == 0) len0 = __builtin_amdgcn_readlane(len[i], seg & 63);
        }
      const int64_t u = T - p - entry;
      blk = u > 0 ? (int32_t)u : 0;
    }
    if (e == 0) {
      w.s = seg;
      w.blk = blk;
    } else {
      w.se = seg;
      w.be = blk;
    }
  }
  return len0;
}

// K operands of one block: TPB tiles of 16 tokens of one page.
template <int TPB> struct KBlock {
  v8i kb[TPB];
  uint32_t ks[TPB]; // MXFP4: E8M0 scale of the lane's block, tile t (byte 0)
  uint32_t ksr;     // FP8: fp32 scale bits of the token this lane stores
  int t0;           // first token of the block
};

// Key bytes and key scales are read once per launch: the loads carry the
// non-temporal hint (cache policy nt), so the stream does not displace the
// small data every launch reuses (lengths, block tables, queries, weights)
// or the logits the top-k reads next (decode scoring 35.6 -> 33.4 us on the
// batched-decode workload, measured).
constexpr int kStream = 2; // buffer-load aux bits: nt

__device__ inline v4i load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStream);
}

__device__ inline uint32_t load4_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kStream);
}

// Physical page of logical page lp of sequence s, or -1 past the table row.
// A scalar load: waiting for it never waits for the K loads in flight.
__device__ inline int64_t page_of(const LogitsArgs &a, int s, int lp) {
  return lp < a.bt_cols ? (int64_t)uniform_load(a.block_tables + (int64_t)s * a.bt_stride + lp) : -1;
}

// Issues the loads of block w.blk of segment w.s. Every tile is loaded, also
// past the segment's end: those rows are inside the page (or read as zeros
// through the buffer bound) and are never stored, and unconditional loads keep
// the wait counts exact so the next block stays in flight during compute.
// With live == false (no next block) the same loads go through empty buffer
// resources: they touch no memory and return zeros, and every path through
// the block loop then has the same number of loads in flight, which keeps the
// compiler's wait counts partial (a path without them would force it to wait
// for every load, including the next block's, before the first MFMA).
// The block's page comes from the caller (pg < 0: nothing to load).
template <int DT, int TPB>
__device__ inline void issue_block_page(const LogitsArgs &a, int blk, int64_t pg,
                                        KBlock<TPB> &kb) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int col = lane & 15;
  const int P = a.page_size;
  const int t0 = blk * a.block_tokens;
  const int lp = t0 / P;
  const int slot0 = t0 - lp * P;
  const bool valid = pg >= 0 && pg < a.num_pages;
  if (!valid) pg = 0;
  const uint32_t page_bytes = (uint32_t)(P * a.row_stride);
  const uint32_t scale_bytes = (uint32_t)((P - 1) * a.scale_row_stride + 4);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(a.kdata + pg * a.page_stride, valid ? page_bytes : 0u);
  const __amdgpu_buffer_rsrc_t sr =
      make_rsrc(a.kscale + pg * a.scale_page_stride, valid ? scale_bytes : 0u);
  kb.t0 = t0;
  if (DT == IDX_FP8_E4M3) {
    // one scale per lane: the token this lane holds after the head-sum
    // reduction (t0 + lane for 4-tile blocks, t0 + 16*(g/2) + col for 2-tile)
    const uint32_t slot = (uint32_t)(slot0 + (TPB == 4 ? lane : 16 * (g >> 1) + col));
    kb.ksr = load4_stream(sr, slot * (uint32_t)a.scale_row_stride);
  }
#pragma unroll
  for (int ti = 0; ti < TPB; ++ti) {
    const uint32_t slot = (uint32_t)(slot0 + ti * kTile + col);
    const uint32_t off = slot * (uint32_t)a.row_stride;
    if (DT == IDX_FP8_E4M3) {
      kb.kb[ti] = cat(load16_stream(kr, off + 16 * g), load16_stream(kr, off + 64 + 16 * g));
    } else {
      const v4i lo = load16_stream(kr, off + 16 * g);
      kb.kb[ti] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
      kb.ks[ti] = load4_stream(sr, slot * (uint32_t)a.scale_row_stride) >> (8 * g);
    }
  }
}

template <int DT, int TPB>
__device__ inline void issue_block(const LogitsArgs &a, const Walk &w, bool live, KBlock<TPB> &kb) {
  const int lp = (w.blk * a.block_tokens) / a.page_size;
  issue_block_page<DT, TPB>(a, w.blk, live ? page_of(a, w.s, lp) : -1, kb);
}

// MFMAs of one 16-token tile against every head tile of every row.
template <int DT, int NROW, int TPB>
__device__ inline void tile_mfma(const QRegs<DT, NROW> &Q, const KBlock<TPB> &kb, int ti,
                                 v4f (&acc)[NROW][4]) {
#pragma unroll
  for (int i = 0; i < NROW; ++i) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const v4f zero = {0.f, 0.f, 0.f, 0.f};
      if (DT == IDX_FP8_E4M3)
        acc[i][m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Q.a[i][m], kb.kb[ti], zero,
                                                                     kFmtFp8, kFmtFp8, 0, 0, 0, 0);
      else
        acc[i][m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            Q.a[i][m], kb.kb[ti], zero, kFmtFp4, kFmtFp4, 0, Q.asc[i][m], 0, (int)kb.ks[ti]);
    }
  }
}

// Logits of up to kStageTokens consecutive tokens per row (one aligned window
// of a segment), staged in LDS and written out 16 bytes per lane: the scores
// of one block are only 256 B per row, and a store that small between the
// K reads costs HBM time far beyond its size.
constexpr int kStageTokens = 256;
template <int NROW> struct OutStage {
  float v[NROW][kStageTokens];
};
struct StageState {
  int base = -1; // first token of the window, -1 when nothing is staged
  int lo = 0;    // staged tokens are [lo, hi)
  int hi = 0;
};

// Writes the staged tokens [lo, min(hi, E, W)) of each row and empties the stage.
template <int DT, int NROW>
__device__ inline void flush_stage(const LogitsArgs &a, const QRegs<DT, NROW> &Q,
                                   const OutStage<NROW> &st, StageState &ss) {
  const int lane = threadIdx.x & 63;
  const int tok = ss.base + 4 * lane; // this lane's four tokens
  const bool vec = (a.W & 3) == 0;    // rows start 16-byte aligned
#pragma unroll
  for (int i = 0; i < NROW; ++i) {
    if (Q.out_row[i] < 0) continue;
    int hi = ss.hi < Q.E[i] ? ss.hi : Q.E[i];
    hi = hi < a.W ? hi : (int)a.W;
    const v4f x = *reinterpret_cast<const v4f *>(&st.v[i][4 * lane]);
    float *row = a.logits + (int64_t)Q.out_row[i] * a.W;
    if (vec && tok >= ss.lo && tok + 4 <= hi) {
      *reinterpret_cast<v4f *>(row + tok) = x;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (tok + j >= ss.lo && tok + j < hi) row[tok + j] = x[j];
    }
  }
  ss.base = -1;
}

// Scores of one loaded block against the segment's rows, staged for logits.
// Tile t+1's MFMAs are issued before tile t's epilogue so the matrix core and
// the vector ALU overlap. Every tile is computed; tokens past the segment's
// end (whose keys may be canary bytes) only reach their own columns and are
// never stored.
template <int DT, int NROW, int TPB>
__device__ inline void score_block(const LogitsArgs &a, const QRegs<DT, NROW> &Q, int32_t L,
                                   const KBlock<TPB> &kb, OutStage<NROW> &st, int base) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int t0 = kb.t0;
  float part[NROW][TPB];
  v4f acc[2][NROW][4];
  tile_mfma<DT, NROW, TPB>(Q, kb, 0, acc[0]);
#pragma unroll
  for (int ti = 0; ti < TPB; ++ti) {
    if (ti + 1 < TPB) tile_mfma<DT, NROW, TPB>(Q, kb, ti + 1, acc[(ti + 1) & 1]);
#pragma unroll
    for (int i = 0; i < NROW; ++i) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) s = fmaf(Q.w[i][m][j], relu2(acc[ti & 1][i][m][j]), s);
      part[i][ti] = s;
    }
  }
  // token held by this lane after the reduction
  const int t = TPB == 4 ? t0 + lane : t0 + 16 * (g >> 1) + (lane & 15);
  const bool holder = TPB == 4 || (g & 1) == 0;
  const int tend = L - t0; // tokens of this block that the segment has
#pragma unroll
  for (int i = 0; i < NROW; ++i) {
    // the head sum of w * 2 relu(s), halved (exact)
    float v = 0.5f * reduce_scatter<TPB>(part[i]);
    // the FP8 key scale of this lane's token is positive, so it commutes with
    // the ReLU and is applied once to the head sum
    if (DT == IDX_FP8_E4M3) v *= __uint_as_float(kb.ksr);
    if (holder && t - t0 < tend) st.v[i][t - base] = v;
  }
}

template <int DT, int NROW>
__device__ inline int32_t enter_segment(const LogitsArgs &a, int s, QRegs<DT, NROW> &Q) {
  int32_t rows[NROW], E[NROW], orow[NROW];
  float qs[NROW];
  const int32_t L = segment_rows<NROW>(a, s, uniform_load(a.lens + s), rows, E, orow);
  load_query<DT, NROW>(Q, a, rows, E, orow, qs);
  return L;
}

// One pipeline step: `cur` holds the loaded current block; the next block's
// loads go into `nxt` before `cur` is scored. Returns false at the end.
template <int DT, int NROW, int TPB>
__device__ inline bool pipeline_step(const LogitsArgs &a, Walk &w, QRegs<DT, NROW> &Q,
                                     int32_t &L, KBlock<TPB> &cur, KBlock<TPB> &nxt,
                                     OutStage<NROW> &st, StageState &ss) {
  Walk wn = w;
  const bool more = advance(a, wn);
  issue_block<DT, TPB>(a, wn, more, nxt);
  if (ss.base < 0) {
    ss.base = cur.t0 & ~(kStageTokens - 1);
    ss.lo = cur.t0;
  }
  score_block<DT, NROW, TPB>(a, Q, L, cur, st, ss.base);
  const int have = L - cur.t0; // tokens of this block that the segment has
  ss.hi = cur.t0 + (have < a.block_tokens ? have : a.block_tokens);
  // the next block continues this window only within the same segment
  if (!more || wn.s != w.s || ((wn.blk * a.block_tokens) & ~(kStageTokens - 1)) != ss.base)
    flush_stage<DT, NROW>(a, Q, st, ss);
  if (!more) return false;
  if (wn.s != w.s) L = enter_segment<DT, NROW>(a, wn.s, Q);
  w = wn;
  return true;
}

template <int DT, int NROW, int TPB>
__global__ __launch_bounds__(64) void mqa_logits_kernel(LogitsArgs a) {
  const int c = blockIdx.x;
  Walk w;
  int32_t len0;
  if (a.cta_info != nullptr) {
    w.s = uniform_load(a.cta_info + 2 * c);
    w.blk = uniform_load(a.cta_info + 2 * c + 1);
    w.s = w.s > 0 ? w.s : 0; // a buffer never written by the builder must not index backwards
    w.blk = w.blk > 0 ? w.blk : 0;
    w.se = uniform_load(a.cta_info + 2 * c + 2);
    w.be = uniform_load(a.cta_info + 2 * c + 3);
    if (!in_range(a, w)) return;
    len0 = segment_length(a, w.s);
  } else {
    len0 = own_range(a, c, w);
    if (!in_range(a, w)) return;
  }
  // The first block's page is read together with the segment's stored
  // length (the table entry exists whether or not the block does). The first
  // segment's queries go out before either returns: their addresses need only
  // the segment, so the query loads, the page lookup and then the first
  // block's K loads overlap, with one wait for all of them.
  const int64_t pg0 = page_of(a, w.s, (w.blk * a.block_tokens) / a.page_size);
  int32_t raw0 = uniform_load(a.lens + w.s);
  w.nb = (len0 + a.block_tokens - 1) >> __builtin_ctz(a.block_tokens);
  const bool stale = w.blk >= w.nb; // empty or stale entry
  if (stale) {
    if (!next_segment(a, w)) return;
    raw0 = uniform_load(a.lens + w.s);
  }
  QRegs<DT, NROW> Q;
  float qs[NROW];
  int32_t L;
  {
    int32_t rows[NROW], E[NROW], orow[NROW];
    L = segment_rows<NROW>(a, w.s, raw0, rows, E, orow);
    load_query<DT, NROW, false>(Q, a, rows, E, orow, qs);
  }
  KBlock<TPB> A, B;
  if (!stale) issue_block_page<DT, TPB>(a, w.blk, pg0, A);
  else issue_block<DT, TPB>(a, w, true, A);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); // the queries and the first block
  scale_weights(Q, qs);
  __shared__ OutStage<NROW> st;
  StageState ss;
  while (pipeline_step<DT, NROW, TPB>(a, w, Q, L, A, B, st, ss) &&
         pipeline_step<DT, NROW, TPB>(a, w, Q, L, B, A, st, ss)) {
  }
}

template <int DT, int NROW, int TPB> hipError_t launch_tpb(const LogitsArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((mqa_logits_kernel<DT, NROW, TPB>), dim3(a.n_ctas), dim3(64), 0, s, a);
  return hipGetLastError();
}

// Blocks of 32 tokens (32-row pages) hold two tiles, larger blocks four.
template <int DT, int NROW> hipError_t launch(const LogitsArgs &a, hipStream_t s) {
  if (a.block_tokens == 32) return launch_tpb<DT, NROW, 2>(a, s);
  if (a.block_tokens == 64) return launch_tpb<DT, NROW, 4>(a, s);
  return hipErrorInvalidValue;
}

template <int DT> hipError_t launch_decode(const LogitsArgs &a, hipStream_t s) {
  switch (a.next_n) {
  case 1: return launch<DT, 1>(a, s);
  case 2: return launch<DT, 2>(a, s);
  case 3: return launch<DT, 3>(a, s);
  case 4: return launch<DT, 4>(a, s);
  default: return hipErrorInvalidValue;
  }
}

} // namespace

hipError_t launch_logits_fp8_decode(const LogitsArgs &a, hipStream_t s) {
  return launch_decode<IDX_FP8_E4M3>(a, s);
}
hipError_t launch_logits_mxfp4_decode(const LogitsArgs &a, hipStream_t s) {
  return launch_decode<IDX_MXFP4>(a, s);
}

} // namespace idx
