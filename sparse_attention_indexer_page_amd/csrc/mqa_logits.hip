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
//   * K is streamed from HBM into a four-slot LDS ring per wave with
//     direct-to-LDS buffer loads, three blocks ahead of the block being
//     scored. Each load instruction fills 1 KB of a slot with whole key rows
//     (eight FP8 rows, sixteen MXFP4 rows), so every 128-byte line of a dense
//     page is read by one instruction; the 16-byte chunks of each row are
//     XOR-swizzled in LDS so that the MFMA operand reads are conflict-free.
//     Versus streaming each block straight into registers one block ahead
//     (the operand order then splits every row over two load instructions),
//     same bits: batched decode 31.0 -> 29.9 us, MTP 43.4 -> 40.4 us, MXFP4
//     unchanged (63-65 us), measured in one run.
//   * One 16-token tile per 16x16x128 MFMA; one MFMA therefore yields 16
//     heads x 16 tokens of full dot products (head_dim 128 = the MFMA's K).
//     FP8 uses the unscaled f8f6f4 form; MXFP4 uses the block-scaled form
//     with the E8M0 scale of each lane's 32-element block as the operand
//     scale.
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
// holds FP8 bytes [16g, 16g+16) and [64+16g, 64+16g+16) of the 128-byte row;
// for MXFP4 it holds bytes [16g, 16g+16) = elements [32g, 32g+32), exactly
// one E8M0 block. Accumulator layout of the 16x16 f32 MFMA: lane l holds
// column (l & 15), rows 4g..4g+3.
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

// Whether ranges are dealt to the XCDs in contiguous eighths (see range_of).
__device__ inline bool xcd_ranges(const LogitsArgs &a) {
  const int n8 = a.n_ctas >> 3;
  return (a.n_ctas & 7) == 0 && (a.lead_ctas == 0 || (n8 & 1) == 0);
}

// The range (schedule entry) that work group c takes. Work groups go to the
// XCDs in turn (c runs on XCD c % 8), so group c takes range
// (c % 8) * (n / 8) + c / 8: each XCD covers one contiguous eighth of the
// work, and a sequence's query and block-table rows are fetched into one
// XCD's L2 rather than all eight (batched decode 31.3 -> 30.9 us, same bits).
__device__ inline int range_of(const LogitsArgs &a, int c) {
  return xcd_ranges(a) ? (c & 7) * (a.n_ctas >> 3) + (c >> 3) : c;
}

// Range r when no schedule buffer is given: the wave computes what the
// schedule builder would write for entries r and r + 1 (same costs:
// ceil(len / BK) blocks per non-empty sequence plus the decode entry cost;
// range r starts at unit floor(r * N / n_ctas) of the N units), from all
// B <= kInlineSplitMaxSegs lengths at once, 64 sequences per lane slot. With
// two work groups per SIMD (lead_ctas > 0) the shares are weighted instead:
// the first lead_ctas groups, dispatched first and one per SIMD, win issue
// arbitration over the second group on their SIMD and take 4/3 of a share
// each (range r starts at floor(cum(r) * N / cum(n_ctas)); with ranges in
// group order cum(r) = 4 min(r, lead) + 3 max(r - lead, 0); MXFP4 decode
// 65.0 -> 63.7 us, MTP 42.1 -> 41.1 us, over a four-copy pool rotation, two
// runs each).
__device__ inline int32_t own_range(const LogitsArgs &a, int r, Walk &w) {
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
  const bool xcd = xcd_ranges(a);
  const int64_t n8 = a.n_ctas >> 3;
  int32_t len0 = 0; // length of the range's first sequence
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    // floor(cum(c + e) N / cum(n_ctas)) through one double division: the
    // numerator (< 2^51; weighted, lead_ctas <= 2^12: < 2^46) and the
    // denominator (<= 2^20) are exact, and a non-integer quotient (< 2^31)
    // lies at least 1/denominator from an integer, far beyond the division's
    // rounding error (< 2^-22), so truncation gives the floor
    const int64_t ce = r + e;
    int64_t num = ce, den = a.n_ctas;
    if (a.lead_ctas > 0 && xcd) {
      // lead_ctas = n / 2: the work groups c < n / 2 take the first half of
      // every XCD's eighth of the ranges
      const int64_t h = n8 >> 1, x = ce / n8, y = ce - x * n8;
      num = 7 * h * x + 4 * (y < h ? y : h) + 3 * (y > h ? y - h : 0);
      den = 7 * h * 8;
    } else if (a.lead_ctas > 0) {
      const int64_t lead = a.lead_ctas;
      num = 4 * (ce < lead ? ce : lead) + 3 * (ce > lead ? ce - lead : 0);
      den = 4 * lead + 3 * (a.n_ctas - lead);
    }
    const int64_t T = (int64_t)((double)(num * N) / (double)den);
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

// One slot of a work group's LDS ring: the key rows of one block, packed at
// the format's row size (128 bytes FP8, 64 bytes MXFP4) with the 16-byte
// chunks of each row XOR-swizzled, then 64 per-token scale words (FP8 fp32;
// MXFP4 four E8M0 bytes, one per 32-element block; words past the page read
// as zeros). Each load instruction fills 1 KB of the image: eight whole FP8
// rows (sixteen MXFP4 rows), so every 128-byte line of a dense page is read
// by one instruction.
template <int DT, int TPB> struct Slot {
  static constexpr int kRowBytes = DT == IDX_FP8_E4M3 ? 128 : 64;
  static constexpr int kUnitsPerRow = kRowBytes / 16;
  static constexpr int kTileBytes = kTile * kRowBytes; // one 16-token tile
  static constexpr int kData = TPB * kTileBytes;
  static constexpr int kDataLoads = kData / 1024;
  static constexpr int kBytes = kData + 256;
  static constexpr int kLoads = kDataLoads + 1; // load instructions per block
};

// Position of chunk c of packed row r within the row: c ^ swizzle(r). Lanes
// (g, col) of an MFMA operand read chunk g (and g + 4) of rows 16t + col; the
// swizzle puts those 16 reads on 16 distinct 16-byte bank groups.
template <int DT> __device__ inline int swizzle(int r) {
  return DT == IDX_FP8_E4M3 ? (r >> 1) & 7 : (r >> 2) & 3;
}


// Physical page of logical page lp of sequence s, or -1 past the table row.
// A scalar load: waiting for it never waits for the K loads in flight. The
// entry is returned as stored (sign-extended only where it is used, so the
// load can stay in flight until then).
__device__ inline int32_t page_of(const LogitsArgs &a, int s, int lp) {
  return lp < a.bt_cols ? uniform_load(a.block_tables + (int64_t)s * a.bt_stride + lp) : -1;
}

__device__ inline int32_t block_page(const LogitsArgs &a, const Walk &w) {
  return page_of(a, w.s, (w.blk * a.block_tokens) >> __builtin_ctz(a.page_size));
}

typedef __attribute__((address_space(3))) void *lds_ptr;

// Buffer resource words (gfx9 raw buffer: base, no stride, size in bytes).
__device__ inline v4i rsrc_words(const void *base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return v4i{(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xffffu), (int)bytes, kRsrcWord3};
}

// Direct-to-LDS loads (16 and 4 bytes per lane): lane l's bytes land at LDS
// address lds + size * l. Key bytes and key scales are read once per launch,
// so the loads carry the non-temporal hint (nt): the stream then does not
// displace the small data every launch reuses (lengths, block tables,
// queries, weights) or the logits the top-k reads next (register-load
// kernel, batched decode: scoring 35.6 -> 33.4 us with the hint, measured). Written as inline assembly so
// that the compiler, which cannot tell which ring slot such a load fills,
// does not wait for every one of them before each LDS read; the scoring loop
// waits for exactly the slot it reads. M0 holds the LDS address; no other
// code of the decode kernel uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm" // m0 in the clobber list
__device__ inline void lds_load16(v4i r, uint32_t lds, uint32_t off, uint32_t soff = 0) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds" ::"s"(lds), "v"(off),
               "s"(r), "s"(soff)
               : "memory", "m0");
}
__device__ inline void lds_load4(v4i r, uint32_t lds, uint32_t off, uint32_t soff = 0) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen nt lds" ::"s"(lds), "v"(off),
               "s"(r), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Lane offsets of a block's loads within its rows: unit j's chunk of row r
// at (r * row_stride + 16 c) and the lane's scale word at (lane * scale row
// stride). The same for every block; the block's first row comes in as the
// instruction's scalar offset.
template <int DT, int TPB> struct SlotOffsets {
  uint32_t data[Slot<DT, TPB>::kDataLoads];
  uint32_t scale;
};

template <int DT, int TPB>
__device__ inline SlotOffsets<DT, TPB> slot_offsets(const LogitsArgs &a) {
  using S = Slot<DT, TPB>;
  const int lane = threadIdx.x & 63;
  SlotOffsets<DT, TPB> o;
#pragma unroll
  for (int j = 0; j < S::kDataLoads; ++j) {
    const int u = 64 * j + lane;       // 16-byte unit of the packed image
    const int r = u / S::kUnitsPerRow; // its row
    const int c = (u % S::kUnitsPerRow) ^ swizzle<DT>(r); // the row's chunk stored there
    o.data[j] = (uint32_t)r * (uint32_t)a.row_stride + 16 * c;
  }
  o.scale = (uint32_t)lane * (uint32_t)a.scale_row_stride;
  return o;
}

// Issues the direct-to-LDS loads of block blk (of page pg; pg < 0: none)
// into a ring slot: always Slot::kLoads instructions, so the wave's count of
// outstanding vector-memory operations tells which slots have landed. With
// no page the loads go through empty buffer resources: they touch no memory
// and leave zeros. Every row of the block is loaded, also past the
// segment's end: those rows are inside the page (or read as zeros through
// the buffer bound) and their scores are never stored. The block's first
// row is the scalar offset: the vector offsets stay below the page's size,
// which is all the bound checks, and the rows read lie inside the page.
template <int DT, int TPB>
__device__ inline void issue_slot(const LogitsArgs &a, const SlotOffsets<DT, TPB> &o, int blk,
                                  int32_t pg, uint8_t *slot) {
  using S = Slot<DT, TPB>;
  const int P = a.page_size;
  const int slot0 = (blk * a.block_tokens) & (P - 1);
  const bool valid = pg >= 0 && pg < a.num_pages;
  const int64_t p = valid ? pg : 0;
  const v4i kr = rsrc_words(a.kdata + p * a.page_stride, valid ? (uint32_t)(P * a.row_stride) : 0u);
  const v4i sr = rsrc_words(a.kscale + p * a.scale_page_stride,
                            valid ? (uint32_t)((P - 1) * a.scale_row_stride + 4) : 0u);
  const uint32_t base = (uint32_t)(uintptr_t)(lds_ptr)slot;
  const uint32_t krow = (uint32_t)slot0 * (uint32_t)a.row_stride;
#pragma unroll
  for (int j = 0; j < S::kDataLoads; ++j) lds_load16(kr, base + 1024 * j, o.data[j], krow);
  lds_load4(sr, base + S::kData, o.scale, (uint32_t)slot0 * (uint32_t)a.scale_row_stride);
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

// Scores of one landed ring slot against the segment's rows, staged for
// logits. Tile t+1's operands are read and its MFMAs issued before tile t's
// epilogue. Every tile is computed; tokens past the segment's end only reach
// their own columns and are never stored.
template <int DT, int NROW, int TPB>
__device__ inline void score_slot(const QRegs<DT, NROW> &Q, int32_t L, int t0, const uint8_t *slot,
                                  OutStage<NROW> &st, int base) {
  using S = Slot<DT, TPB>;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int col = lane & 15;
  // row 16t + col's swizzle does not depend on the tile t
  const int lo = S::kRowBytes * col + 16 * (g ^ swizzle<DT>(col));
  const int hi = lo ^ 64; // chunk g + 4 (FP8)
  auto operand = [&](int ti, v8i &b, uint32_t &bs) {
    const uint8_t *p = slot + S::kTileBytes * ti;
    if (DT == IDX_FP8_E4M3) {
      b = cat(*reinterpret_cast<const v4i *>(p + lo), *reinterpret_cast<const v4i *>(p + hi));
    } else {
      const v4i x = *reinterpret_cast<const v4i *>(p + lo);
      b = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
      bs = *reinterpret_cast<const uint32_t *>(slot + S::kData + 4 * (kTile * ti + col)) >> (8 * g);
    }
  };
  auto mfma = [&](const v8i &b, uint32_t bs, v4f (&acc)[NROW][4]) {
#pragma unroll
    for (int i = 0; i < NROW; ++i) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
        if (DT == IDX_FP8_E4M3)
          acc[i][m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Q.a[i][m], b, zero, kFmtFp8,
                                                                       kFmtFp8, 0, 0, 0, 0);
        else
          acc[i][m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              Q.a[i][m], b, zero, kFmtFp4, kFmtFp4, 0, Q.asc[i][m], 0, (int)bs);
      }
    }
  };
  float part[NROW][TPB];
  v4f acc[2][NROW][4];
  v8i b[2];
  uint32_t bs[2] = {0u, 0u};
  operand(0, b[0], bs[0]);
  mfma(b[0], bs[0], acc[0]);
#pragma unroll
  for (int ti = 0; ti < TPB; ++ti) {
    if (ti + 1 < TPB) {
      operand(ti + 1, b[(ti + 1) & 1], bs[(ti + 1) & 1]);
      mfma(b[(ti + 1) & 1], bs[(ti + 1) & 1], acc[(ti + 1) & 1]);
    }
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
  const int tl = TPB == 4 ? lane : 16 * (g >> 1) + col;
  const bool holder = TPB == 4 || (g & 1) == 0;
  float ks = 1.f;
  if (DT == IDX_FP8_E4M3) ks = *reinterpret_cast<const float *>(slot + S::kData + 4 * tl);
#pragma unroll
  for (int i = 0; i < NROW; ++i) {
    // the head sum of w * 2 relu(s), halved (exact)
    float v = 0.5f * reduce_scatter<TPB>(part[i]);
    // the FP8 key scale of this lane's token is positive, so it commutes with
    // the ReLU and is applied once to the head sum
    if (DT == IDX_FP8_E4M3) v *= ks;
    if (holder && tl < L - t0) st.v[i][t0 + tl - base] = v;
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

// The first segment's query rows are staged through the ring's last slots:
// per row the codes (64 heads x 128 FP8 bytes or 64 MXFP4 bytes), MXFP4's
// E8M0 block scales (64 x 4 bytes) and the 64 fp32 weights.
template <int DT> struct QStage {
  static constexpr int kCodes = kHeads * (DT == IDX_FP8_E4M3 ? kHeadDim : kHeadDim / 2);
  static constexpr int kScales = DT == IDX_FP8_E4M3 ? 0 : kHeads * (kHeadDim / 32);
  static constexpr int kRow = kCodes + kScales + kHeads * 4;
  static constexpr int kLoads = kCodes / 1024 + (DT == IDX_FP8_E4M3 ? 0 : 1) + 1; // per row
};

// Slots the first segment's staged queries occupy, or 0 when they take more
// than two: those query rows are loaded into registers before the ring starts
// (a round trip more at start-up, but an LDS ring of four slots, which keeps
// eight work groups on a CU).
template <int DT, int NROW, int TPB> constexpr int query_slots() {
  constexpr int qs = (NROW * QStage<DT>::kRow + Slot<DT, TPB>::kBytes - 1) / Slot<DT, TPB>::kBytes;
  return qs <= 2 ? qs : 0;
}

// Ring slots per work group: four (17-34 KB of LDS, so 4-8 groups share a CU).
constexpr int kRingSlots = decode_ring_slots();

// Issues the direct-to-LDS loads of a segment's query rows (rows[i] < 0:
// zeros) into the staging area at lds.
template <int DT, int NROW>
__device__ inline void issue_query(const LogitsArgs &a, const int32_t (&rows)[NROW], uint8_t *lds) {
  using Q = QStage<DT>;
  const int lane = threadIdx.x & 63;
  const uint32_t base = (uint32_t)(uintptr_t)(lds_ptr)lds;
#pragma unroll
  for (int i = 0; i < NROW; ++i) {
    const bool live = rows[i] >= 0;
    const int64_t r = live ? rows[i] : 0;
    const uint32_t row = base + i * Q::kRow;
    const v4i qr = rsrc_words(a.q + r * Q::kCodes, live ? (uint32_t)Q::kCodes : 0u);
#pragma unroll
    for (int j = 0; j < Q::kCodes / 1024; ++j) lds_load16(qr, row + 1024 * j, 1024 * j + 16 * lane);
    if (DT != IDX_FP8_E4M3) {
      const v4i sr = rsrc_words(a.q_scale + r * Q::kScales, live ? (uint32_t)Q::kScales : 0u);
      lds_load4(sr, row + Q::kCodes, 4 * lane);
    }
    const v4i wr = rsrc_words(a.weights + r * kHeads, live ? (uint32_t)(kHeads * 4) : 0u);
    lds_load4(wr, row + Q::kCodes + Q::kScales, 4 * lane);
  }
}

// Reads staged query rows into the MFMA A operands and the lane's weights.
template <int DT, int NROW>
__device__ inline void read_query(QRegs<DT, NROW> &Q, const uint8_t *lds, const int32_t (&E)[NROW],
                                  const int32_t (&out_rows)[NROW]) {
  using S = QStage<DT>;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int hl = lane & 15;
#pragma unroll
  for (int i = 0; i < NROW; ++i) {
    Q.E[i] = E[i];
    Q.out_row[i] = out_rows[i];
    const uint8_t *row = lds + i * S::kRow;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int h = 16 * m + hl;
      if (DT == IDX_FP8_E4M3) {
        const v4i *p = reinterpret_cast<const v4i *>(row + h * kHeadDim);
        Q.a[i][m] = cat(p[g], p[4 + g]);
      } else {
        const v4i lo = *reinterpret_cast<const v4i *>(row + h * (kHeadDim / 2) + 16 * g);
        Q.a[i][m] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
        Q.asc[i][m] = row[S::kCodes + h * (kHeadDim / 32) + g];
      }
      const v4f wv = *reinterpret_cast<const v4f *>(row + S::kCodes + S::kScales + 4 * (16 * m + 4 * g));
#pragma unroll
      for (int j = 0; j < 4; ++j) Q.w[i][m][j] = wv[j];
    }
  }
}

// One wave per work group. The wave streams its range's key blocks into an
// LDS ring with direct-to-LDS loads, R - 1 blocks ahead of the block it
// scores: a second walk over the same range (the load walk) issues block
// i + R - 1 into the slot block i - 1 vacated, then the wave waits until at
// most (R - 1) blocks' loads are outstanding, which (vector-memory loads
// complete in issue order) means block i has landed. The wave's other
// vector-memory operations only make that wait longer, never shorter: the
// logits stores come after the loads they could overtake, and a segment's
// query loads are waited for in full.
template <int DT, int NROW, int TPB>
__global__ __launch_bounds__(64) void mqa_logits_kernel(LogitsArgs a) {
  using S = Slot<DT, TPB>;
  constexpr int R = kRingSlots;
  constexpr int QS = query_slots<DT, NROW, TPB>(); // staging slots of the first queries
  __shared__ __attribute__((aligned(16))) uint8_t ring[R][S::kBytes];
  __shared__ OutStage<NROW> st;
  static_assert(sizeof(ring) + sizeof(st) ==
                    decode_lds_bytes(DT == IDX_FP8_E4M3, TPB * kTile, NROW),
                "the recommended work-group count assumes this LDS size");
  const int c = range_of(a, blockIdx.x);
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
  // segment's queries go out (into the ring's last QS slots) before the first
  // blocks' loads, one wait covers the queries and the first block, and the
  // staging slots then receive the next blocks. Every load of the wave goes
  // straight to LDS, so the compiler has no register loads of its own to wait
  // for (such a wait would also wait for the ring).
  int32_t pgl = block_page(a, w);
  int32_t raw0 = uniform_load(a.lens + w.s);
  w.nb = (len0 + a.block_tokens - 1) >> __builtin_ctz(a.block_tokens);
  if (w.blk >= w.nb) { // empty or stale entry
    if (!next_segment(a, w)) return;
    raw0 = uniform_load(a.lens + w.s);
    pgl = block_page(a, w);
  }
  QRegs<DT, NROW> Q;
  float qs[NROW];
  int32_t L;
  int32_t rows[NROW], E[NROW], orow[NROW];
  L = segment_rows<NROW>(a, w.s, raw0, rows, E, orow);
  Walk wl = w;      // load walk: the next block to issue, of page pgl
  bool more_l = true;
  int sl = 0;       // its ring slot
  const SlotOffsets<DT, TPB> so = slot_offsets<DT, TPB>(a);
  auto issue_next = [&]() {
    issue_slot<DT, TPB>(a, so, wl.blk, more_l ? pgl : -1, ring[sl]);
    sl = sl + 1 == R ? 0 : sl + 1;
    if (more_l) {
      more_l = advance(a, wl);
      if (more_l) pgl = block_page(a, wl);
    }
  };
  if constexpr (QS > 0) {
#pragma unroll
    for (int i = 0; i < NROW; ++i)
      qs[i] = DT == IDX_FP8_E4M3 && a.q_scale != nullptr && rows[i] >= 0
                  ? uniform_load(reinterpret_cast<const float *>(a.q_scale) + rows[i])
                  : 1.f;
    issue_query<DT, NROW>(a, rows, ring[R - QS]);
#pragma unroll
    for (int j = 0; j < R - QS; ++j) issue_next();
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((R - QS - 1) * S::kLoads)); // the queries and block 0
    read_query<DT, NROW>(Q, ring[R - QS], E, orow);
    scale_weights(Q, qs);
    // the staging slots are read before the next blocks' loads overwrite them
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
#pragma unroll
    for (int j = R - QS; j < R - 1; ++j) issue_next();
  } else {
    // the first block goes out first, so the query loads' full wait covers
    // it and the key stream is not held back by the query round trip; the
    // other blocks follow the wait, so the CU's start-up burst is the
    // queries and one block per wave (MTP scoring 41.5 -> 40.9 us against
    // all three blocks first, 41.2 with none and 40.9 with two)
    issue_next();
    load_query<DT, NROW>(Q, a, rows, E, orow, qs); // loaded and waited for
#pragma unroll
    for (int j = 1; j < R - 1; ++j) issue_next();
  }
  StageState ss;
  int sc = 0; // ring slot of the block scored next
  while (true) {
    issue_next();
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((R - 1) * S::kLoads));
    const int t0 = w.blk * a.block_tokens;
    if (ss.base < 0) {
      ss.base = t0 & ~(kStageTokens - 1);
      ss.lo = t0;
    }
    score_slot<DT, NROW, TPB>(Q, L, t0, ring[sc], st, ss.base);
    sc = sc + 1 == R ? 0 : sc + 1;
    const int have = L - t0; // tokens of this block that the segment has
    ss.hi = t0 + (have < a.block_tokens ? have : a.block_tokens);
    Walk wn = w;
    const bool more = advance(a, wn);
    // the next block continues this window only within the same segment
    if (!more || wn.s != w.s || ((wn.blk * a.block_tokens) & ~(kStageTokens - 1)) != ss.base)
      flush_stage<DT, NROW>(a, Q, st, ss);
    if (!more) break;
    if (wn.s != w.s) L = enter_segment<DT, NROW>(a, wn.s, Q);
    w = wn;
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
