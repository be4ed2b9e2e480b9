// Work split of the paged scoring kernel, built on the device in one launch.
//
// ROCm/ATOM PR #1709 ("Add fp4 indexer fo dsv4"), commit on
// compute_varctx_schedule: building the decode schedule with many small
// launches plus an allocation and a copy cost ~300 us per step; one kernel
// writing straight into the fixed-address buffer a captured graph reads cut
// it to ~40 us. This builder is that single launch: it reads the current
// lengths on the device (so a graph replay after an in-place length update
// sees the new lengths) and writes every work group's start coordinate.
//
// A segment (a sequence in decode, a block of query rows in prefill) of
// length L owns ceil(L / BK) blocks of BK = min(page_size, 64) tokens; BK
// divides the page size, so a block never straddles two physical pages
// (vllm-project/DeepGEMM PR #14: BLOCK_KV = min(PAGE_KV, 64)). Blocks of all
// segments, in order, form one list; a non-empty segment also carries a fixed
// entry cost (its query load) of `entry_cost` units in front of its blocks.
// The list is cut into n_ctas contiguous ranges of equal cost (to one unit).
// Entry c of the buffer is (segment, block) of range c's first block -- a
// start inside a segment's entry units is that segment's block 0, so two
// ranges may share a start and the first of them is empty; entry n_ctas is
// (nseg, 0).
#include "internal.h"

namespace idx {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ inline int32_t segment_length(const ScheduleArgs &a, int s) {
  if (a.mode == kSegDecode) return clamp_seg_len(a.lens[s]);
  int32_t m = 0;
  const int r0 = a.row0 + s * kPrefillRowsPerSeg;
#pragma unroll
  for (int i = 0; i < kPrefillRowsPerSeg; ++i) {
    const int r = r0 + i;
    if (r < a.row_end) {
      const int32_t v = a.lens[r];
      m = v > m ? v : m;
    }
  }
  m = clamp_seg_len(m);
  return m <= a.skip_len ? 0 : m; // rows that select all their keys need no scores
}

__global__ __launch_bounds__(kThreads) void schedule_kernel(ScheduleArgs a) {
  if (a.mode == kSegPrefill && a.n_chunks > 1) { // this work group's chunk
    const int g = blockIdx.x;
    a.row0 += g * a.chunk_rows;
    const int32_t end = a.row0 + a.chunk_rows;
    a.row_end = end < a.row_end ? end : a.row_end;
    a.nseg = (a.row_end - a.row0 + kPrefillRowsPerSeg - 1) / kPrefillRowsPerSeg;
    a.cta_info += g * a.chunk_ints;
  }
  // prefix[s] = cost of segments [0, s)
  extern __shared__ int32_t prefix[];
  __shared__ int32_t wave_tot[kWaves];
  __shared__ int32_t carry;
  __shared__ int32_t total;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();

  for (int base = 0; base < a.nseg; base += kThreads) {
    const int s = base + tid;
    int32_t nb = 0;
    if (s < a.nseg) {
      const int32_t L = segment_length(a, s);
      nb = (L + a.block_tokens - 1) / a.block_tokens;
      if (nb > 0) nb += a.entry_cost;
    }
    int32_t incl = nb; // inclusive scan within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
      int32_t v = lane < kWaves ? wave_tot[lane] : 0;
#pragma unroll
      for (int off = 1; off < kWaves; off <<= 1) {
        const int32_t y = __shfl_up(v, off, 64);
        if (lane >= off) v += y;
      }
      if (lane < kWaves) wave_tot[lane] = v; // inclusive over waves
    }
    __syncthreads();
    const int32_t c0 = carry;
    const int32_t before = c0 + (wave ? wave_tot[wave - 1] : 0) + incl - nb;
    if (s < a.nseg) prefix[s] = before;
    __syncthreads();
    if (tid == 0) carry = c0 + wave_tot[kWaves - 1];
    __syncthreads();
  }
  if (tid == 0) total = carry;
  __syncthreads();

  const int64_t N = total;
  for (int c = tid; c <= a.n_ctas; c += kThreads) {
    const int64_t start = (c == a.n_ctas) ? N : ((int64_t)c * N) / a.n_ctas;
    int32_t seg, blk;
    if (start >= N) {
      seg = a.nseg;
      blk = 0;
    } else {
      // last s with prefix[s] <= start; segment s then contains unit `start`
      int lo = 0, hi = a.nseg;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (prefix[mid] <= start) lo = mid;
        else hi = mid;
      }
      seg = lo;
      const int64_t u = start - prefix[lo] - a.entry_cost;
      blk = u > 0 ? (int32_t)u : 0;
    }
    a.cta_info[2 * c] = seg;
    a.cta_info[2 * c + 1] = blk;
  }
}

// Per-row visible ends of a ragged decode step (ROCm/ATOM PR #1709, commits
// on the ragged varlen windows: each sequence's draft rows see a window that
// ends at its committed length and moves every step, so it is rebuilt on the
// device each step; a rectangular step is the uniform case). Sequence b owns
// rows [off[b], off[b+1]), at most max_q of them; its row j sees
// len_b - (n_b - 1 - j) keys. Every row of the [B * max_q] buffer is written:
// rows no sequence owns get 0, so a fixed-shape top-k over the whole buffer
// selects nothing for them.
// Visible length of row r: with offsets, the ragged rule above (0 for a row
// no sequence owns); without, row r = b*n + j of the rectangular step.
__device__ inline int32_t row_window(const int32_t *lens, const int32_t *off, int32_t B,
                                     int32_t n_max, int64_t r) {
  if (off == nullptr) {
    const int64_t b = r / n_max;
    const int32_t j = (int32_t)(r - b * n_max);
    const int32_t e = lens[b] - (n_max - 1 - j);
    return e > 0 ? e : 0;
  }
  // last sequence b with off[b] <= r (offsets are non-decreasing)
  if (off[0] > r) return 0;
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= r) lo = mid;
    else hi = mid;
  }
  const int32_t base = off[lo];
  int32_t n = off[lo + 1] - base;
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  const int32_t j = (int32_t)(r - base);
  if (j >= n) return 0;
  const int32_t len = lens[lo] > 0 ? lens[lo] : 0;
  const int32_t e = len - (n - 1 - j);
  return e > 0 ? e : 0;
}

__global__ __launch_bounds__(256) void varlen_windows_kernel(const int32_t *lens,
                                                             const int32_t *off, int32_t B,
                                                             int32_t max_q, int32_t *ve) {
  const int64_t rows = (int64_t)B * max_q;
  for (int64_t r = blockIdx.x * 256ll + threadIdx.x; r < rows; r += (int64_t)gridDim.x * 256)
    ve[r] = row_window(lens, off, B, max_q, r);
}

// -inf into columns [E_r, W) of every row of a [B * n][W] logits buffer (the
// opt-in that makes the whole buffer defined). Work group (x, y): row y,
// columns [1024 x, 1024 x + 1024), four per thread.
__global__ __launch_bounds__(256) void fill_tail_kernel(const int32_t *lens, const int32_t *off,
                                                        int32_t B, int32_t n, int64_t W,
                                                        float *logits) {
  const int64_t r = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * 1024 + 4 * threadIdx.x;
  if (t0 >= W) return;
  int64_t e = row_window(lens, off, B, n, r);
  e = e < W ? e : W;
  float *row = logits + r * W;
  const float ninf = -__builtin_huge_valf();
  if ((W & 3) == 0 && t0 >= e && t0 + 4 <= W) {
    *reinterpret_cast<float4 *>(row + t0) = float4{ninf, ninf, ninf, ninf};
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (t0 + i >= e && t0 + i < W) row[t0 + i] = ninf;
  }
}

} // namespace

hipError_t launch_varlen_windows(const int32_t *lens, const int32_t *row_offsets, int32_t B,
                                 int32_t max_q, int32_t *visible_end, hipStream_t s) {
  const int64_t rows = (int64_t)B * max_q;
  const int64_t g = (rows + 255) / 256;
  hipLaunchKernelGGL(varlen_windows_kernel, dim3(g < 1024 ? (unsigned)g : 1024u), dim3(256), 0,
                     s, lens, row_offsets, B, max_q, visible_end);
  return hipGetLastError();
}

hipError_t launch_fill_tail(const int32_t *lens, const int32_t *row_offsets, int32_t B, int32_t n,
                            int64_t W, float *logits, hipStream_t s) {
  const int64_t gx = (W + 1023) / 1024;
  hipLaunchKernelGGL(fill_tail_kernel, dim3((unsigned)gx, (unsigned)(B * n)), dim3(256), 0, s,
                     lens, row_offsets, B, n, W, logits);
  return hipGetLastError();
}

hipError_t launch_schedule(const ScheduleArgs &a, hipStream_t s) {
  const size_t lds = sizeof(int32_t) * (size_t)(a.nseg > 0 ? a.nseg : 1);
  hipLaunchKernelGGL(schedule_kernel, dim3(a.n_chunks > 1 ? a.n_chunks : 1), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

} // namespace idx
