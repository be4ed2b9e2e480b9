// Prefill scores of the sparse-attention indexer on gfx950.
//
//   logits[r][t] = sum_h w[r][h] * max(0, k_scale[t] * (q[r][h] . k[t])),  t < visible_end[r]
//
// Prefill scores many query rows of one sequence against the same committed
// keys (ROCm/ATOM PR #1709, commit on right-sizing the prefill logits: rows
// see [0, visible_end) of a right-sized width, processed in Q-row chunks). Here
// the work is a dense heads x tokens contraction per row that reuses every
// key block across rows, so the kernel is built around key reuse:
//   * A work group of 16 waves (one per CU, four per SIMD) owns a block of 15
//     consecutive query rows: 15 compute waves hold one row's q each (the MFMA
//     A operands, in VGPRs), and one loader wave streams the key blocks of the
//     schedule's item range into a 6-slot LDS ring with direct-to-LDS buffer
//     loads; the waves score two key blocks between barriers, with two more
//     pairs in flight. Every key block is read from L2 once per 15 rows.
//     Versus two 8-wave groups of 7 rows per CU (same occupancy, same bits):
//     the L2 -> LDS key traffic halves and the longer chunk of the 16384-row
//     prefill takes 217.9 instead of 222-224 us on average over 23 calls, its
//     clock-throttled peak 227 instead of 234-237 us (kernel traces, two
//     alternating runs).
//   * Only the loader wave issues the LDS loads and it stores nothing, so its
//     vector-memory counter counts exactly those loads: it waits for the stage
//     about to be consumed, then one barrier publishes it to the compute waves
//     and frees the stage consumed last, which the loader refills.
//   * Loads are bounded by each page's buffer resource (a block-table entry
//     outside the pool reads zeros), and blocks of BK = min(P, 64) tokens never
//     straddle a page (vllm-project/DeepGEMM PR #14: BLOCK_KV = min(PAGE_KV, 64)).
//   * Compute per 16-token tile: operands straight from LDS in MFMA lane order
//     (each lane reads the 16 bytes it needs, conflict-free), 4 MFMAs over the
//     64 heads (FP8: 16x16x128; MXFP4: block-scaled), the same fused ReLU /
//     weight / head-sum epilogue and lane-group reduce-scatter as decode: the
//     ReLU is taken doubled (x + |x|, one full-rate add) and the head sum is
//     halved once per token, which is exact.
#include "device_common.h"
#include "internal.h"

namespace idx {
namespace {

using namespace dev;

constexpr int kWaves = kPrefillRowsPerSeg + 1;
constexpr int kRowsPerGroup = kWaves - 1; // compute waves, one query row each
constexpr int kGroup = 2;           // key blocks scored between two barriers
constexpr int kStages = 3 * kGroup; // ring slots: one group in use, two in flight
constexpr int kLoader = kWaves - 1; // the loader wave's index
static_assert(kRowsPerGroup == kPrefillRowsPerSeg, "schedule segments are the row blocks");

template <int DT, int TPB> struct Stage {
  // FP8: tile t's half h (bytes [64h, 64h+64) of each row) in chunk 2t+h;
  // MXFP4: tile t in chunk t. A chunk is 64 lanes x 16 B in MFMA lane order.
  static constexpr int kChunks = DT == IDX_FP8_E4M3 ? 2 * TPB : TPB;
  static constexpr int kData = kChunks * 1024;
  static constexpr int kBytes = kData + 256; // + one 4-byte scale word per token
  static constexpr int kLoads = kChunks + 1; // loader instructions per stage
};

template <int L> __device__ inline void wait_loads_outstanding(int items) {
  // at most `items` later stages (L loads each) may still be in flight
  static_assert(kGroup == 2 && 2 * L < 64, "one immediate per possible count");
  if (items <= 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  else if (items == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(L));
  else __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * L));
}

// Work-group barrier for the stage ring. __syncthreads (and even an LDS-only
// fence, since direct-to-LDS loads count as vector-memory ops) waits for every
// outstanding vector-memory op, which would drain the loader's prefetched
// stages and stall compute waves on their logits stores. Here the loader has
// already waited for exactly the stage being published, compute waves only
// read LDS, and LDS ops are waited for (lgkmcnt) before the barrier; the
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct Walk {
  int s, blk, se, be, nb;
};

__device__ inline int32_t block_length(const LogitsArgs &a, int s) {
  int32_t L = 0;
#pragma unroll
  for (int i = 0; i < kRowsPerGroup; ++i) {
    const int r = a.row0 + s * kRowsPerGroup + i;
    if (r < a.row_end) {
      const int32_t e = uniform_load(a.lens + r);
      L = e > L ? e : L;
    }
  }
  L = clamp_seg_len(L);
  // a block whose rows all select every visible key needs no scores (the
  // schedule builder applies the same rule)
  return L <= a.skip_len ? 0 : L;
}

__device__ inline bool in_range(const LogitsArgs &a, const Walk &w) {
  return w.s < a.nseg && (w.s < w.se || (w.s == w.se && w.blk < w.be));
}

__device__ inline bool next_segment(const LogitsArgs &a, Walk &w) {
  w.blk = 0;
  while (true) {
    ++w.s;
    if (!in_range(a, w)) return false;
    w.nb = (block_length(a, w.s) + a.block_tokens - 1) / a.block_tokens;
    if (w.nb > 0) return true;
  }
}

__device__ inline bool advance(const LogitsArgs &a, Walk &w) {
  if (++w.blk < w.nb) return in_range(a, w);
  return next_segment(a, w);
}

// Loader wave: key block w.blk into a stage (data chunks, then scale words).
template <int DT, int TPB>
__device__ inline void load_stage(const LogitsArgs &a, const Walk &w, uint8_t *stage) {
  using S = Stage<DT, TPB>;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int col = lane & 15;
  const int P = a.page_size;
  const int t0 = w.blk * a.block_tokens;
  const int lp = t0 / P;
  const int slot0 = t0 - lp * P;
  int64_t pg = lp < a.bt_cols ? (int64_t)uniform_load(a.block_tables + lp) : -1;
  const bool valid = pg >= 0 && pg < a.num_pages;
  if (!valid) pg = 0;
  const __amdgpu_buffer_rsrc_t kr =
      make_rsrc(a.kdata + pg * a.page_stride, valid ? (uint32_t)(P * a.row_stride) : 0u);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(
      a.kscale + pg * a.scale_page_stride, valid ? (uint32_t)((P - 1) * a.scale_row_stride + 4) : 0u);
#pragma unroll
  for (int c = 0; c < S::kChunks; ++c) {
    const int tile = DT == IDX_FP8_E4M3 ? c >> 1 : c;
    const int half = DT == IDX_FP8_E4M3 ? c & 1 : 0;
    const uint32_t off = (uint32_t)(slot0 + kTile * tile + col) * (uint32_t)a.row_stride + 64 * half + 16 * g;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (__attribute__((address_space(3))) void *)(stage + 1024 * c),
                                             16, off, 0, 0, 0);
  }
  // scale word of token slot0 + lane (lanes past the page read zeros)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      sr, (__attribute__((address_space(3))) void *)(stage + S::kData), 4,
      (uint32_t)(slot0 + lane) * (uint32_t)a.scale_row_stride, 0, 0, 0);
}

struct Row {
  v8i a[4];       // A operands of the four head tiles
  int32_t asc[4]; // MXFP4 E8M0 scale of the lane's block
  float w[4][4];  // weights of the lane's 16 heads (times the FP8 q scale)
  int32_t lim;    // tokens of the row stored: min(visible length, W); 0 for a padding row
  float *orow;    // the row's logits (wave-uniform, so the store address is scalar + lane)
};

template <int DT> __device__ inline void enter_block(const LogitsArgs &a, int s, Row &R) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int hl = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = a.row0 + s * kRowsPerGroup + wave;
  if (r >= a.row_end) {
    R.lim = 0;
    R.orow = a.logits;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      R.a[m] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      R.asc[m] = 127;
#pragma unroll
      for (int j = 0; j < 4; ++j) R.w[m][j] = 0.f;
    }
    return;
  }
  const int32_t e = uniform_load(a.lens + r);
  // the block's length is the clamped maximum over its rows, so this never
  // passes the last block scored
  const int32_t ec = clamp_seg_len(e);
  R.lim = ec < a.W ? ec : (int32_t)a.W;
  R.orow = a.logits + (int64_t)(r - a.row0) * a.W;
  float qs = 1.f;
  if (DT == IDX_FP8_E4M3 && a.q_scale != nullptr) qs = uniform_load(reinterpret_cast<const float *>(a.q_scale) + r);
  const float *wrow = a.weights + (int64_t)r * kHeads;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int h = 16 * m + hl;
    if (DT == IDX_FP8_E4M3) {
      const v4i *p = reinterpret_cast<const v4i *>(a.q + ((int64_t)r * kHeads + h) * kHeadDim);
      R.a[m] = cat(p[g], p[4 + g]);
    } else {
      const v4i *p = reinterpret_cast<const v4i *>(a.q + ((int64_t)r * kHeads + h) * (kHeadDim / 2));
      const v4i lo = p[g];
      R.a[m] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
      R.asc[m] = a.q_scale[((int64_t)r * kHeads + h) * (kHeadDim / 32) + g];
    }
    const v4f wv = *reinterpret_cast<const v4f *>(wrow + 16 * m + 4 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) R.w[m][j] = wv[j] * qs;
  }
  // Wait for the q loads here, once per row block: left outstanding, the
  // compiler's wait for them at their first use would be a full vmcnt(0) in
  // every pass of the stage loop, i.e. a wait for the wave's logits stores.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// Compute wave: scores of one staged key block against its row.
template <int DT, int TPB>
__device__ inline void score_stage(const Row &R, const uint8_t *stage, int t0) {
  using S = Stage<DT, TPB>;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int col = lane & 15;
  float part[TPB];
  v4f acc[2][4];
  v8i b[2];
  uint32_t bs[2] = {0u, 0u};
  auto operand = [&](int ti, v8i &bv, uint32_t &bsv) {
    if (DT == IDX_FP8_E4M3) {
      bv = cat(*reinterpret_cast<const v4i *>(stage + 1024 * (2 * ti) + 16 * lane),
               *reinterpret_cast<const v4i *>(stage + 1024 * (2 * ti + 1) + 16 * lane));
    } else {
      const v4i lo = *reinterpret_cast<const v4i *>(stage + 1024 * ti + 16 * lane);
      bv = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
      bsv = *reinterpret_cast<const uint32_t *>(stage + S::kData + 4 * (kTile * ti + col)) >> (8 * g);
    }
  };
  auto mfma = [&](int ti, v4f (&ac)[4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const v4f zero = {0.f, 0.f, 0.f, 0.f};
      if (DT == IDX_FP8_E4M3)
        ac[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(R.a[m], b[ti & 1], zero, kFmtFp8,
                                                                 kFmtFp8, 0, 0, 0, 0);
      else
        ac[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(R.a[m], b[ti & 1], zero, kFmtFp4,
                                                                 kFmtFp4, 0, R.asc[m], 0, (int)bs[ti & 1]);
    }
  };
  operand(0, b[0], bs[0]);
  mfma(0, acc[0]);
#pragma unroll
  for (int ti = 0; ti < TPB; ++ti) {
    if (ti + 1 < TPB) {
      operand(ti + 1, b[(ti + 1) & 1], bs[(ti + 1) & 1]);
      mfma(ti + 1, acc[(ti + 1) & 1]);
    }
    float sum = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) sum = fmaf(R.w[m][j], relu2(acc[ti & 1][m][j]), sum);
    part[ti] = sum;
  }
  float v = 0.5f * reduce_scatter<TPB>(part);
  const int tl = TPB == 4 ? lane : kTile * (g >> 1) + col; // token of this lane in the block
  if (DT == IDX_FP8_E4M3) v *= *reinterpret_cast<const float *>(stage + S::kData + 4 * tl);
  const int t = t0 + tl;
  const bool holder = TPB == 4 || (g & 1) == 0;
  if (holder && t < R.lim) R.orow[t] = v;
}

template <int DT, int TPB>
__global__ __launch_bounds__(kWaves * 64, 1) void prefill_logits_kernel(LogitsArgs a) {
  using S = Stage<DT, TPB>;
  __shared__ __attribute__((aligned(16))) uint8_t ring[kStages][S::kBytes];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); // wave-uniform
  const bool loader = wave == kLoader;
  const int c = blockIdx.x;

  Walk w;
  w.s = uniform_load(a.cta_info + 2 * c);
  w.blk = uniform_load(a.cta_info + 2 * c + 1);
  w.s = w.s > 0 ? w.s : 0; // a buffer never written by the builder must not index backwards
  w.blk = w.blk > 0 ? w.blk : 0;
  w.se = uniform_load(a.cta_info + 2 * c + 2);
  w.be = uniform_load(a.cta_info + 2 * c + 3);
  if (!in_range(a, w)) return;
  w.nb = (block_length(a, w.s) + a.block_tokens - 1) / a.block_tokens;
  if (w.blk >= w.nb && !next_segment(a, w)) return; // empty or stale entry
  // every wave holds the same walk, so all reach the same barriers

  Walk wl = w; // loader: the next block to load
  bool more_l = true;
  int issued = 0; // blocks issued by the loader; block b goes to slot b % kStages
  if (loader) {
    for (int st = 0; st < 2 * kGroup && more_l; ++st) {
      load_stage<DT, TPB>(a, wl, ring[st]);
      ++issued;
      more_l = advance(a, wl);
    }
  }
  Row R;
  if (!loader) enter_block<DT>(a, w.s, R);

  // Group i scores blocks [i G, i G + G) from their slots. Before its barrier
  // the loader waits for those blocks (the next group's may stay in flight);
  // after it, the slots of group i - 1 are free and receive group i + 2.
  for (int i = 0;; ++i) {
    if (loader) wait_loads_outstanding<S::kLoads>(issued - (i + 1) * kGroup);
    lds_barrier();
    if (loader) {
      for (int u = 0; u < kGroup && more_l; ++u) {
        load_stage<DT, TPB>(a, wl, ring[issued % kStages]);
        ++issued;
        more_l = advance(a, wl);
      }
    }
    bool done = false;
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      if (!loader) score_stage<DT, TPB>(R, ring[(i * kGroup + u) % kStages], w.blk * a.block_tokens);
      const int s_prev = w.s;
      if (!advance(a, w)) {
        done = true;
        break;
      }
      if (w.s != s_prev && !loader) enter_block<DT>(a, w.s, R);
    }
    if (done) break;
  }
}

template <int DT> hipError_t launch(const LogitsArgs &a, hipStream_t s) {
  if (a.block_tokens == 32) {
    hipLaunchKernelGGL((prefill_logits_kernel<DT, 2>), dim3(a.n_ctas), dim3(kWaves * 64), 0, s, a);
  } else if (a.block_tokens == 64) {
    hipLaunchKernelGGL((prefill_logits_kernel<DT, 4>), dim3(a.n_ctas), dim3(kWaves * 64), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

} // namespace

hipError_t launch_logits_fp8_prefill(const LogitsArgs &a, hipStream_t s) {
  return launch<IDX_FP8_E4M3>(a, s);
}
hipError_t launch_logits_mxfp4_prefill(const LogitsArgs &a, hipStream_t s) {
  return launch<IDX_MXFP4>(a, s);
}

} // namespace idx
