// Per-row top-k of the indexer scores on gfx950 ("indexer_score_topk" in
// ROCm/ATOM PR #1709 "Add fp4 indexer fo dsv4", commit on the forward_pre /
// score_topk_from split). Row r selects the min(k, E_r) token indices with the
// largest scores among t < E_r; equal scores go to the lower index; the
// indices are written in ascending order and the rest of the row is -1.
//
// One work group per row holds the whole row in registers (up to 65536
// scores: 16 waves x 64 lanes x 64). Scores become order-preserving uint32
// keys (-0 folded onto +0). The exact k-th largest key is found by radix
// select: the first digit is the top 11 bits of (key - min key) over the
// row's actual key range, so the histogram spreads over the occupied range
// instead of piling into a handful of exponent bins; further 11-bit digits
// refine inside the chosen bin until one key value remains or the bin fills
// the remaining quota exactly. Histograms live in LDS. Selection then walks
// the row in index order: wave w owns a contiguous segment, each round covers
// 64 consecutive indices, and ballot/popcount give every selected lane its
// output slot, so no sort is needed and ties resolve to the lower index.
#include "internal.h"

namespace idx {
namespace {

constexpr int kBins = 2048;
constexpr int kDigitBits = 11;

__device__ inline uint32_t float_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0; // -0 == +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ inline uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

__device__ inline uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(v, off, 64);
    v = o < v ? o : v;
  }
  return v;
}

__device__ inline int32_t wave_sum_i32(int32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Count of set lanes below this lane in a 64-bit ballot.
__device__ inline int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

template <int NT, int IPT>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
  constexpr int NW = NT / 64;
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t red_u[2 * NW];
  __shared__ int32_t red_i[2 * NW];
  __shared__ uint32_t s_sel[4]; // bin, count above bin, count in bin
  if (threadIdx.x < 4) s_sel[threadIdx.x] = 0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = blockIdx.x;
  const int b = r / a.next_n;
  const int j = r - b * a.next_n;
  int64_t E = (int64_t)a.lens[b] - (a.next_n - 1 - j);
  if (E < 0) E = 0;
  if (E > a.W) E = a.W;
  const int k = a.k;
  int32_t *out = a.out_idx + (int64_t)r * k;
  if (a.out_count && tid == 0) a.out_count[r] = (int32_t)(E < k ? E : k);

  if (E <= k) { // everything visible is selected
    for (int i = tid; i < k; i += NT) out[i] = i < E ? i : -1;
    return;
  }

  // wave segment of seg_len indices (a multiple of 64), IPT rounds at most
  const int rounds = (int)((E + (int64_t)NW * 64 - 1) / ((int64_t)NW * 64));
  const int seg_len = rounds * 64;
  const int base = wave * seg_len;
  const float *row = a.logits + (int64_t)r * a.W;

  uint32_t key[IPT];
  uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int idx = base + i * 64 + lane;
    key[i] = 0; // 0 = not a visible index (every finite score maps above 0x007FFFFF)
    if (i < rounds && idx < E) {
      key[i] = float_key(row[idx]);
      kmax = key[i] > kmax ? key[i] : kmax;
      kmin = key[i] < kmin ? key[i] : kmin;
    }
  }
  kmax = wave_max_u32(kmax);
  kmin = wave_min_u32(kmin);
  if (lane == 0) {
    red_u[wave] = kmax;
    red_u[NW + wave] = kmin;
  }
  __syncthreads();
  kmax = 0;
  kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    kmax = red_u[w] > kmax ? red_u[w] : kmax;
    kmin = red_u[NW + w] < kmin ? red_u[NW + w] : kmin;
  }

  // Radix select over (key - lo) within [lo, lo + 2^shift * kBins).
  uint32_t lo = kmin;           // every candidate key is >= lo
  uint32_t span = kmax - kmin;  // candidates lie in [lo, lo + span]
  int32_t need = k;             // how many of the candidates to take
  uint32_t thr = 0;             // final threshold key
  int32_t need_eq = 0;          // how many keys == thr to take (lowest indices)
  bool done = false;
  while (!done) {
    if (span == 0) { // one key value left
      thr = lo;
      need_eq = need;
      break;
    }
    const int bits = 32 - __clz(span);
    const int shift = bits > kDigitBits ? bits - kDigitBits : 0;
    for (int i = tid; i < kBins; i += NT) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      if (i < rounds && key[i] >= lo && key[i] - lo <= span)
        atomicAdd(&hist[(key[i] - lo) >> shift], 1u);
    }
    __syncthreads();
    // Find bin d* (from the top) where the running count reaches `need`.
    if (wave == 0) {
      constexpr int PER = kBins / 64;
      // lane owns bins kBins-1-lane*PER down to kBins-PER-lane*PER
      const int top = kBins - 1 - lane * PER;
      uint32_t mine = 0;
#pragma unroll 8
      for (int q = 0; q < PER; ++q) mine += hist[top - q];
      // inclusive prefix over lanes (lane 0 = highest bins)
      uint32_t incl = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      const uint32_t excl = incl - mine;
      if (excl < (uint32_t)need && incl >= (uint32_t)need) {
        uint32_t run = excl;
        for (int q = 0; q < PER; ++q) {
          const uint32_t cq = hist[top - q];
          if (run + cq >= (uint32_t)need) {
            s_sel[0] = (uint32_t)(top - q);
            s_sel[1] = run;
            s_sel[2] = cq;
            break;
          }
          run += cq;
        }
      }
    }
    __syncthreads();
    const uint32_t d = s_sel[0];
    const int32_t above = (int32_t)s_sel[1];
    const int32_t inbin = (int32_t)s_sel[2];
    __syncthreads(); // s_sel and hist are rewritten by the next pass
    need -= above;
    const uint32_t blo = lo + (d << shift);
    if (inbin == need) { // the whole bin fits: take every key >= blo
      thr = blo - 1u;    // blo >= min visible key >= 0x00800000, so no wrap
      need_eq = 0;
      done = true;
      break;
    }
    lo = blo;
    const uint32_t width = shift >= 32 ? 0xFFFFFFFFu : ((1u << shift) - 1u);
    span = (kmax - lo) < width ? (kmax - lo) : width;
  }

  // Index-ordered selection: key > thr always; key == thr for the first
  // need_eq such indices.
  int32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    if (i < rounds) {
      const bool valid = key[i] != 0;
      n_gt += (valid && key[i] > thr) ? 1 : 0;
      n_eq += (valid && key[i] == thr) ? 1 : 0;
    }
  }
  n_gt = wave_sum_i32(n_gt);
  n_eq = wave_sum_i32(n_eq);
  if (lane == 0) {
    red_i[wave] = n_gt;
    red_i[NW + wave] = n_eq;
  }
  __syncthreads();
  int32_t gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) {
    gt_before += red_i[w];
    eq_before += red_i[NW + w];
  }
  int32_t pos = gt_before + (eq_before < need_eq ? eq_before : need_eq);
  int32_t eq_seen = eq_before;
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    if (i < rounds) {
      const bool valid = key[i] != 0;
      const bool gt = valid && key[i] > thr;
      const bool eq = valid && key[i] == thr;
      const uint64_t meq = __ballot(eq);
      const int eq_rank = eq_seen + lanes_below(meq);
      const bool sel = gt || (eq && eq_rank < need_eq);
      const uint64_t msel = __ballot(sel);
      const int p = pos + lanes_below(msel);
      if (sel && p < k) out[p] = base + i * 64 + lane;
      pos += __popcll(msel);
      eq_seen += __popcll(meq);
    }
  }
}

template <int NT, int IPT> hipError_t launch_rows(const TopkArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((topk_kernel<NT, IPT>), dim3(a.R), dim3(NT), 0, s, a);
  return hipGetLastError();
}

} // namespace

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
  if (a.W <= 4096) return launch_rows<256, 16>(a, s);
  if (a.W <= 16384) return launch_rows<512, 32>(a, s);
  return launch_rows<1024, 64>(a, s);
}

} // namespace idx
