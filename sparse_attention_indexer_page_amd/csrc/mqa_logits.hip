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
//     then a two-step cross-lane sum over the four lane groups; the FP8
//     per-token K scale and per-row q scale are positive, so they are applied
//     outside the ReLU (relu(s*x) = s*relu(x) for s >= 0).
//
// Operand lane layout (identical for A and B, which is all a full-length dot
// product needs): lane l serves row/column (l & 15); lane group g = l >> 4
// holds FP8 bytes [16g, 16g+16) and [64+16g, 64+16g+16) of the 128-byte row,
// so each of the two 16-byte loads of a 16-row tile reads 64 contiguous bytes
// per row; for MXFP4 it holds bytes [16g, 16g+16) = elements [32g, 32g+32),
// exactly one E8M0 block. Accumulator layout of the 16x16 f32 MFMA: lane l
// holds column (l & 15), rows 4g..4g+3.
#include "internal.h"

namespace idx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kFmtFp8 = 0; // f8f6f4 format code: E4M3
constexpr int kFmtFp4 = 4; // f8f6f4 format code: E2M1

// Raw buffer resource word 3 for gfx9: no swizzle, no format conversion.
constexpr int kRsrcWord3 = 0x00020000;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

__device__ inline v4i load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ inline uint32_t load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

__device__ inline v8i cat(v4i a, v4i b) { return v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}; }

__device__ inline float lane_xor_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// Query-side registers of one segment.
template <int DT, int NROW> struct QRegs {
  v8i a[NROW][4];    // A operands per row and head tile
  int32_t asc[NROW][4]; // MXFP4: E8M0 scale of the lane's block (byte 0)
  float w[NROW][4][4];  // weight (times FP8 q scale) of the lane's 16 heads
  int32_t E[NROW];      // visible length per row
  int32_t out_row[NROW]; // logits row, or -1 for a padding row
};

template <int DT, int NROW>
__device__ inline void load_query(QRegs<DT, NROW> &Q, const LogitsArgs &a, const int32_t *rows,
                                  const int32_t *E, const int32_t *out_rows) {
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
      continue;
    }
    float qs = 1.f;
    if (DT == IDX_FP8_E4M3 && a.q_scale != nullptr)
      qs = reinterpret_cast<const float *>(a.q_scale)[r];
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
      for (int j = 0; j < 4; ++j) Q.w[i][m][j] = wv[j] * qs;
    }
  }
}

// Rows, visible lengths and output rows of segment s; returns its length.
template <int NROW, bool PREFILL>
__device__ inline int32_t segment_rows(const LogitsArgs &a, int s, int32_t *rows, int32_t *E,
                                       int32_t *out_rows) {
  int32_t L = 0;
#pragma unroll
  for (int i = 0; i < NROW; ++i) {
    if (PREFILL) {
      const int r = a.row0 + s * NROW + i;
      const bool ok = r < a.row_end;
      int32_t e = ok ? a.lens[r] : 0;
      e = e > 0 ? e : 0;
      rows[i] = ok ? r : -1;
      E[i] = e;
      out_rows[i] = ok ? r - a.row0 : -1;
      L = e > L ? e : L;
    } else {
      const int r = s * a.next_n + i;
      int32_t e = a.lens[s] - (a.next_n - 1 - i);
      e = e > 0 ? e : 0;
      rows[i] = r;
      E[i] = e;
      out_rows[i] = r;
      L = e > L ? e : L;
    }
  }
  return L;
}

template <int DT, int NROW, bool PREFILL>
__global__ __launch_bounds__(64) void mqa_logits_kernel(LogitsArgs a) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int col = lane & 15;
  const int c = blockIdx.x;

  int s = a.cta_info[2 * c];
  int blk = a.cta_info[2 * c + 1];
  s = s > 0 ? s : 0; // a buffer never written by the builder must not index backwards
  blk = blk > 0 ? blk : 0;
  const int se = a.cta_info[2 * c + 2];
  const int be = a.cta_info[2 * c + 3];

  const int P = a.page_size;
  const int BK = a.block_tokens;
  const uint32_t page_bytes = (uint32_t)(P * a.row_stride);
  const uint32_t scale_bytes = (uint32_t)((P - 1) * a.scale_row_stride + 4);

  QRegs<DT, NROW> Q;
  int cur = -1;
  int32_t L = 0, nb = 0;
  const int32_t *bt = a.block_tables;

  while (s < a.nseg && (s < se || (s == se && blk < be))) {
    if (s != cur) {
      int32_t rows[NROW], E[NROW], orow[NROW];
      L = segment_rows<NROW, PREFILL>(a, s, rows, E, orow);
      nb = (L + BK - 1) / BK;
      if (blk >= nb) { // empty segment or a stale schedule: move on
        ++s;
        blk = 0;
        continue;
      }
      load_query<DT, NROW>(Q, a, rows, E, orow);
      bt = a.block_tables + (int64_t)s * a.bt_stride;
      cur = s;
    }

    // ---- one block: up to BK/16 tiles of one page
    const int t0 = blk * BK;
    const int lp = t0 / P;
    const int slot0 = t0 - lp * P;
    int64_t pg = lp < a.bt_cols ? (int64_t)bt[lp] : -1;
    const bool valid = pg >= 0 && pg < a.num_pages;
    if (!valid) pg = 0;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(a.kdata + pg * a.page_stride, valid ? page_bytes : 0u);
    const int tend = (L - t0) < BK ? (L - t0) : BK;
    const int ntile = (tend + kTile - 1) / kTile;

    v8i kb[4];
    uint32_t ks[4];
    if (DT == IDX_FP8_E4M3) {
      const __amdgpu_buffer_rsrc_t sr =
          make_rsrc(a.kscale + pg * a.scale_page_stride, valid ? scale_bytes : 0u);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        if (ti < ntile) {
          const uint32_t slot = (uint32_t)(slot0 + ti * kTile + col);
          const uint32_t off = slot * (uint32_t)a.row_stride;
          kb[ti] = cat(load16(kr, off + 16 * g), load16(kr, off + 64 + 16 * g));
          ks[ti] = load4(sr, slot * (uint32_t)a.scale_row_stride);
        }
      }
    } else {
      const __amdgpu_buffer_rsrc_t sr =
          make_rsrc(a.kscale + pg * a.scale_page_stride, valid ? scale_bytes : 0u);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        if (ti < ntile) {
          const uint32_t slot = (uint32_t)(slot0 + ti * kTile + col);
          const v4i lo = load16(kr, slot * (uint32_t)a.row_stride + 16 * g);
          kb[ti] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
          ks[ti] = load4(sr, slot * (uint32_t)a.scale_row_stride) >> (8 * g);
        }
      }
    }

    float outv[NROW];
#pragma unroll
    for (int i = 0; i < NROW; ++i) outv[i] = 0.f;

#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      if (ti < ntile) {
#pragma unroll
        for (int i = 0; i < NROW; ++i) {
          float part = 0.f;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            v4f acc = {0.f, 0.f, 0.f, 0.f};
            if (DT == IDX_FP8_E4M3)
              acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Q.a[i][m], kb[ti], acc, kFmtFp8,
                                                                     kFmtFp8, 0, 0, 0, 0);
            else
              acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  Q.a[i][m], kb[ti], acc, kFmtFp4, kFmtFp4, 0, Q.asc[i][m], 0, (int)ks[ti]);
#pragma unroll
            for (int j = 0; j < 4; ++j) part = fmaf(Q.w[i][m][j], fmaxf(acc[j], 0.f), part);
          }
          part = lane_xor_sum(part);
          if (DT == IDX_FP8_E4M3) part *= __uint_as_float(ks[ti]);
          if (g == ti) outv[i] = part;
        }
      }
    }

    // lane l now holds token t0 + l (tile g, column col) of every row
    const int t = t0 + lane;
#pragma unroll
    for (int i = 0; i < NROW; ++i) {
      if (Q.out_row[i] >= 0 && lane < tend && t < Q.E[i] && t < a.W)
        a.logits[(int64_t)Q.out_row[i] * a.W + t] = outv[i];
    }

    if (++blk >= nb) {
      ++s;
      blk = 0;
    }
  }
}

template <int DT, int NROW, bool PREFILL>
hipError_t launch(const LogitsArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((mqa_logits_kernel<DT, NROW, PREFILL>), dim3(a.n_ctas), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int DT> hipError_t launch_decode(const LogitsArgs &a, hipStream_t s) {
  switch (a.next_n) {
  case 1: return launch<DT, 1, false>(a, s);
  case 2: return launch<DT, 2, false>(a, s);
  case 3: return launch<DT, 3, false>(a, s);
  case 4: return launch<DT, 4, false>(a, s);
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
hipError_t launch_logits_fp8_prefill(const LogitsArgs &a, hipStream_t s) {
  return launch<IDX_FP8_E4M3, kPrefillRowsPerSeg, true>(a, s);
}
hipError_t launch_logits_mxfp4_prefill(const LogitsArgs &a, hipStream_t s) {
  return launch<IDX_MXFP4, kPrefillRowsPerSeg, true>(a, s);
}

} // namespace idx
