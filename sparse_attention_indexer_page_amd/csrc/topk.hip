// Per-row top-k of the indexer scores on gfx950 ("indexer_score_topk" in
// ROCm/ATOM PR #1709 "Add fp4 indexer fo dsv4", commit on the forward_pre /
// score_topk_from split). Row r selects the min(k, E_r) token indices with the
// largest scores among t < E_r; equal scores go to the lower index; the
// indices are written in ascending order and the rest of the row is -1.
//
// Two kernels, chosen by the logits width W. Up to W = 4096 (prefill widths)
// one wave owns a row, with no work-group barrier (see below). Wider rows
// take one work group per row; the row's keys stay in registers. Scores become
// order-preserving uint32 keys (-0 folded onto +0); the number of keys per
// lane is a compile-time bucket chosen from the row's actual length, so every
// loop is fully unrolled and all loads of the row are in flight at once. The
// exact k-th largest key is found by radix select on 12/12/8-bit digits (top
// bits first): the first digit's histogram covers every key; the keys in the
// chosen bin (typically a few hundred) are then compacted into LDS and only
// they are refined, until one key value remains or a bin fills the remaining
// quota exactly. Histograms live in LDS; the bin holding the k-th key is found
// with a block-wide scan. Selection walks the row in index order: wave w owns
// a contiguous segment, a counting pass gives each wave its output offset, and
// a writing pass uses ballot/popcount per 64 indices, so no sort is needed and
// ties resolve to the lower index. When every key equal to the threshold is
// taken (the common case) both passes reduce to one comparison per key.
#include "device_common.h"
#include "internal.h"

namespace idx {
namespace {

using namespace dev;

constexpr int kBins = 4096;
constexpr int kDigitBits = 12;

__device__ inline uint32_t float_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0; // -0 == +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inverse of float_key (for keys of finite scores).
__device__ inline float key_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Sum over the wave's 64 lanes, in every lane, without LDS: quad swaps, the
// half-row and row mirrors (DPP), then the gfx950 row swaps.
__device__ inline uint32_t wave_sum(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, false); // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0u, v, 0x140, 0xF, 0xF, false); // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = a[0] + a[1];
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return b[0] + b[1];
}

// Max / min over the wave's 64 lanes, in every lane, the same way.
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x140, 0xF, 0xF, false));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(b[0], b[1]);
}
__device__ inline uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x140, 0xF, 0xF, false));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = min(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return min(b[0], b[1]);
}

// Inclusive prefix sum over the wave's lanes with DPP moves: shifts by 1, 2,
// 4, 8 within each 16-lane row (lanes shifted in from outside the row add
// 0), then row 0's total into rows 1 and 3 and row 1's into rows 2 and 3
// (row_bcast 15), then the first half's into the second (row_bcast 31).
__device__ inline uint32_t wave_incl_scan_u32(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xF, 0xF, false); // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xF, 0xF, false); // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, false); // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xF, 0xF, false); // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xA, 0xF, false); // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xC, 0xF, false); // row_bcast:31
  return v;
}

// Count of set lanes below this lane in a 64-bit ballot.
__device__ inline int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Smallest key in (lo, hi] whose bin (a monotone non-decreasing function of
// the key) is at least b, given that hi's is: a 64-way search, each lane
// testing one evenly spaced key per round (at most six rounds for 32-bit
// keys). lo itself is never evaluated. Wave-uniform result.
template <typename BinOf>
__device__ __forceinline__ uint32_t first_key_in_bin_at_least(uint32_t lo, uint32_t hi, uint32_t b,
                                                             BinOf bin_of) {
  const int lane = threadIdx.x & 63;
  while (hi - lo > 1u) {
    const uint32_t step = (hi - lo + 63u) / 64u;
    const uint32_t off = (uint32_t)(lane + 1) * step; // <= hi - lo + 63: no wrap below 2^32
    const uint32_t x = off >= hi - lo ? hi : lo + off;
    const uint64_t m = __ballot(bin_of(x) >= b); // false ... false, true ... true (lane 63: hi)
    const int f = (int)__builtin_ctzll(m);
    const uint32_t nhi = __builtin_amdgcn_readlane(x, f);
    lo = f == 0 ? lo : __builtin_amdgcn_readlane(x, f - 1);
    hi = nhi;
  }
  return hi;
}

// The same search, first tried over the 64 keys just below and above
// `guess` (a key computed to lie near the answer): the narrower interval is
// taken only where the bins at its ends confirm that it holds the answer,
// so the result is the same, in one round instead of up to six.
template <typename BinOf>
__device__ __forceinline__ uint32_t first_key_in_bin_near(uint32_t lo, uint32_t hi, uint32_t b,
                                                         uint32_t guess, BinOf bin_of) {
  constexpr uint32_t kHalf = 32u;
  if (guess > lo + kHalf && guess - kHalf < hi && bin_of(guess - kHalf) < b) lo = guess - kHalf;
  if (hi > kHalf && guess < hi - kHalf && guess + kHalf > lo && bin_of(guess + kHalf) >= b)
    hi = guess + kHalf;
  return first_key_in_bin_at_least(lo, hi, b, bin_of);
}

// A key near the lower edge of value bin b under the linear map
// bin = (x / 2 - h0) * scale (the edge's value, rounded).
__device__ inline uint32_t bin_edge_key(uint32_t b, float h0, float scale) {
  return float_key(((float)b / scale + h0) * 2.0f);
}

constexpr int kCandCap = 4096; // keys of the first pass's bin refined in LDS

constexpr int kRankCap = 64; // candidates ranked directly by one wave

struct TopkShared {
  uint32_t hist[kBins];
  uint32_t cand[kCandCap];
  uint32_t cidx[kCandCap]; // row index of cand[i] when the candidates are a sampled threshold's
  uint32_t small[kRankCap];
  uint32_t red[3 * 16];
  uint32_t ered[2 * 16]; // the output's per-wave counts (their own, so no
                         // barrier has to separate them from reads of red)
  uint32_t sel[3]; // bin, count above it, count in it
  uint32_t ncand;
  uint32_t nsmall;
};

// Histogram of digit(key) over the keys accepted by `in`, then the bin that
// holds the need-th largest: returns (bin, count above it, count in it).
// The histogram is all zero on entry (cleared at the start of the row, and
// each pass clears the bins it reads), so a pass takes three barriers: the
// first also orders every earlier read of red and sel before this pass
// writes them.
template <int NT, typename Visit>
__device__ __forceinline__ void radix_pass(TopkShared &sm, int need, Visit visit, uint32_t &bin,
                                  int &above, int &inbin) {
  constexpr int NW = NT / 64;
  constexpr int BPT = kBins / NT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  visit([&](uint32_t d) { atomicAdd(&sm.hist[d], 1u); });
  __syncthreads();
  // Block-wide scan from the highest bin down: thread t owns bins
  // [kBins-1-t*BPT, kBins-1-(t+1)*BPT), and clears them for the next pass
  // (whose first add follows this pass's last barrier).
  const int top = kBins - 1 - tid * BPT;
  uint32_t cnt[BPT];
  uint32_t mine = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    cnt[q] = sm.hist[top - q];
    sm.hist[top - q] = 0u;
    mine += cnt[q];
  }
  const uint32_t incl = wave_incl_scan_u32(mine);
  if (lane == 63) sm.red[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) before += w < wave ? sm.red[w] : 0u;
  const uint32_t excl = before + incl - mine;
  if (excl < (uint32_t)need && excl + mine >= (uint32_t)need) {
    uint32_t run = excl;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      if (run < (uint32_t)need && run + cnt[q] >= (uint32_t)need) {
        sm.sel[0] = (uint32_t)(top - q);
        sm.sel[1] = run;
        sm.sel[2] = cnt[q];
      }
      run += cnt[q];
    }
  }
  __syncthreads();
  bin = sm.sel[0];
  above = (int)sm.sel[1];
  inbin = (int)sm.sel[2];
}

// Block-wide max and min of per-thread values and sum of per-wave counts
// (wave-uniform `cnt`); uniform results. The first use of red in the work
// group: nothing has read it before.
template <int NT>
__device__ __forceinline__ void block_max_min(TopkShared &sm, uint32_t &mx, uint32_t &mn,
                                              uint32_t &cnt) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  mx = wave_max_u32(mx);
  mn = wave_min_u32(mn);
  if (lane == 0) {
    sm.red[wave] = mx;
    sm.red[16 + wave] = mn;
    sm.red[32 + wave] = cnt;
  }
  __syncthreads();
  mx = 0u;
  mn = 0xFFFFFFFFu;
  cnt = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mx = sm.red[w] > mx ? sm.red[w] : mx;
    mn = sm.red[16 + w] < mn ? sm.red[16 + w] : mn;
    cnt += sm.red[32 + w];
  }
}

// Writes the selection in index order, given the rule found: every key >
// thr, and of the keys == thr the first need_eq (all of them when all_ties;
// then the rule is key >= thr_ge). Each wave owns N consecutive runs of 64
// items; item q of this lane has key key_at(q) (0: nothing) and row index
// idx_at(q), increasing with the wave, q and the lane. A counting pass gives
// each wave its output offset, a writing pass places the indices with
// ballots, so no sort is needed and ties go to the lower index.
template <int NT, int N, typename KeyAt, typename IdxAt>
__device__ __forceinline__ void emit_selection(TopkShared &sm, KeyAt key_at, IdxAt idx_at,
                                               uint32_t thr, int need_eq, bool all_ties,
                                               uint32_t thr_ge, int k, int32_t *out) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // ---- counting pass: per wave, keys taken wholesale and keys == thr
  uint32_t n_gt = 0, n_eq = 0;
  if (all_ties) {
#pragma unroll
    for (int i = 0; i < N; ++i) n_gt += __popcll(__ballot(key_at(i) >= thr_ge));
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) { // key 0 (no item) never reaches thr
      const uint32_t x = key_at(i);
      n_gt += __popcll(__ballot(x > thr));
      n_eq += __popcll(__ballot(x == thr));
    }
  }
  if (lane == 0) {
    sm.ered[wave] = n_gt;
    sm.ered[16 + wave] = n_eq;
  }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    gt_before += w < wave ? (int)sm.ered[w] : 0;
    eq_before += w < wave ? (int)sm.ered[16 + w] : 0;
  }

  // ---- writing pass in index order (the comparisons are made again rather
  // than kept from the counting pass: 2 N ballots held across its barriers
  // would not fit the scalar registers)
  asm volatile("" : "+v"(thr), "+v"(thr_ge));
  if (all_ties) {
    int pos = gt_before;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bool sel = key_at(i) >= thr_ge;
      const uint64_t msel = __ballot(sel);
      const int p = pos + lanes_below(msel);
      if (sel && p < k) out[p] = idx_at(i);
      pos += (int)__popcll(msel);
    }
  } else {
    int pos = gt_before + (eq_before < need_eq ? eq_before : need_eq);
    int eq_seen = eq_before;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint32_t x = key_at(i);
      const bool eq = x == thr;
      const uint64_t meq = __ballot(eq);
      const bool sel = x > thr || (eq && eq_seen + lanes_below(meq) < need_eq);
      const uint64_t msel = __ballot(sel);
      const int p = pos + lanes_below(msel);
      if (sel && p < k) out[p] = idx_at(i);
      pos += (int)__popcll(msel);
      eq_seen += (int)__popcll(meq);
    }
  }
}

// The exact selection over candidates compacted into LDS in index order:
// sm.cand[0, nc) holds their raw score bits (keyed here, as they are read)
// and sm.cidx their row indices (both complete since a barrier before the
// call); every key of the row >= lo is among them; k <= nc of them are taken.
// hi >= lo is a key of the row (the largest of a sample): the first pass bins
// [lo, hi] by key bits and puts every key beyond its top bin into that bin,
// so the bins stay key intervals (the top one open above). Refines by key
// bits within the chosen interval (radix passes over the LDS candidates, then
// one wave ranks the last few) and writes the selection in index order.
template <int NT>
__device__ __forceinline__ void select_compacted(TopkShared &sm, int nc, uint32_t lo, uint32_t hi,
                                                 int k, int32_t ib, int32_t *out) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int need = k, cand = nc;
  uint32_t thr;    // final rule: key > thr, plus need_eq keys == thr (lowest index first)
  int need_eq = 0; // 0: every key >= thr + 1 is taken
  int n_eq_total = -1;
  bool open = true; // keys above hi may remain (first pass only)
  while (true) {
    if (!open && lo == hi) { // a single key value
      thr = lo;
      need_eq = need;
      n_eq_total = cand;
      break;
    }
    if (cand <= kRankCap) {
      // one wave ranks the candidates: lane l holds candidate l (on the first
      // pass every compacted key is one, so hi is not used)
      const bool direct = cand == nc; // every compacted key is a candidate
      if (!direct) {
        for (int c0 = wave * 64; c0 < nc; c0 += NT) {
          const int c = c0 + lane;
          const uint32_t x = c < nc ? float_key(__uint_as_float(sm.cand[c])) : 0u;
          const bool in = c < nc && x >= lo && x <= hi;
          const uint64_t m = __ballot(in);
          if (m) {
            uint32_t at = 0;
            if (lane == 0) at = atomicAdd(&sm.nsmall, (uint32_t)__popcll(m));
            at = __builtin_amdgcn_readlane(at, 0);
            if (in) sm.small[at + lanes_below(m)] = x;
          }
        }
        __syncthreads();
      }
      if (wave == 0) {
        const uint32_t mykey =
            lane < cand ? (direct ? float_key(__uint_as_float(sm.cand[lane])) : sm.small[lane]) : 0u;
        int gt = 0, eq = 0;
        for (int j = 0; j < cand; ++j) {
          const uint32_t x = __builtin_amdgcn_readlane(mykey, j);
          gt += x > mykey ? 1 : 0;
          eq += x == mykey ? 1 : 0;
        }
        const bool is_thr = lane < cand && gt < need && gt + eq >= need;
        const int tl = (int)__builtin_ctzll(__ballot(is_thr));
        if (lane == tl) {
          sm.sel[0] = mykey;
          sm.sel[1] = (uint32_t)(need - gt);
          sm.sel[2] = (uint32_t)eq;
        }
      }
      __syncthreads();
      thr = sm.sel[0];
      need_eq = (int)sm.sel[1];
      n_eq_total = (int)sm.sel[2];
      break;
    }
    const uint32_t range = hi - lo;
    const int bits = range != 0u ? 32 - __builtin_clz(range) : 0;
    const int shift = bits > kDigitBits ? bits - kDigitBits : 0;
    uint32_t bin;
    int above, inbin;
    radix_pass<NT>(
        sm, need,
        [&](auto add) {
          for (int c = tid; c < nc; c += NT) {
            const uint32_t x = float_key(__uint_as_float(sm.cand[c]));
            if (x >= lo && (open || x <= hi)) {
              const uint32_t d = (x - lo) >> shift; // < kBins unless open
              add(d < (uint32_t)kBins ? d : (uint32_t)(kBins - 1));
            }
          }
        },
        bin, above, inbin);
    need -= above;
    cand = inbin;
    const uint32_t nlo = lo + (bin << shift);
    const uint32_t width = (1u << shift) - 1u;
    if (open) // a bin below the top is the whole interval; the top one is open
      hi = bin == (uint32_t)(kBins - 1) ? 0xFFFFFFFFu : nlo + width;
    else
      hi = hi - nlo < width ? hi : nlo + width;
    open = false;
    lo = nlo;
    if (inbin == need) { // the whole bin is taken
      thr = lo - 1u;
      break;
    }
  }
  // every key equal to thr is taken: the rule is key >= thr_ge
  const bool all_ties = need_eq == 0 || need_eq == n_eq_total;
  const uint32_t thr_ge = need_eq == 0 ? thr + 1u : thr;
  // over the compacted keys: wave w owns entries [w * run, w * run + run)
  constexpr int NQ = kCandCap / NT; // runs of 64 per wave (run <= kCandCap / NW)
  static_assert(kCandCap % NT == 0, "whole runs per wave");
  const int run = (((nc + NW - 1) / NW) + 63) & ~63;
  const int j0 = wave * run + lane;
  emit_selection<NT, NQ>(
      sm,
      [&](int q) -> uint32_t {
        const int j = j0 + 64 * q;
        return 64 * q < run && j < nc ? float_key(__uint_as_float(sm.cand[j])) : 0u;
      },
      [&](int q) -> int32_t { return ib + (int32_t)sm.cidx[j0 + 64 * q]; }, thr, need_eq, all_ties,
      thr_ge, k, out);
}

// Whether a score's key is >= thr, from its raw bits b alone. Above +0's key
// (POS) the passing scores are the positive ones with b >= thr - 2^31 (b read
// as a signed integer: negative scores are negative). Below it they are every
// score of sign 0 and the negative ones with ~b >= thr, i.e. b <= ~thr
// unsigned, which every sign-0 b satisfies too (~thr >= 2^31), and so does -0
// (0x80000000), as its key is +0's. Raw 0, the value of a slot past the row,
// passes exactly when thr is below +0's key.
template <bool POS> __device__ inline bool raw_at_least(uint32_t b, uint32_t thr) {
  return POS ? (int32_t)b >= (int32_t)(thr & 0x7FFFFFFFu) : b <= ~thr;
}

// The exact count of the row's keys >= thr (over every wave's IPT raw scores
// per lane, row index base + 64 i + lane; slots past the row hold 0) and,
// when it lies in [k, kCandCap], the compaction of those scores' raw bits and
// indices into LDS in index order, then the selection over them. Returns
// whether the selection was made (else nothing is written and the caller runs
// the full passes). Slots past the row that pass (only when thr is below +0's
// key) have the highest indices, so they take the last positions and are
// left out.
template <int NT, int IPT, bool POS>
__device__ __forceinline__ bool count_compact(TopkShared &sm, const uint32_t (&b)[IPT], uint32_t thr,
                                              uint32_t smax, int E, int k, int base, int32_t ib,
                                              int32_t *out) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t n0 = 0;
#pragma unroll
  for (int i = 0; i < IPT; ++i) n0 += (uint32_t)__popcll(__ballot(raw_at_least<POS>(b[i], thr)));
  if (lane == 0) sm.red[wave] = n0;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    before += w < wave ? sm.red[w] : 0u;
    total += sm.red[w];
  }
  if (!POS) total -= (uint32_t)(NT * IPT - E); // the slots past the row all pass
  if (total < (uint32_t)k || total > (uint32_t)kCandCap) return false;
  uint32_t at = before;
  // the comparisons are made again rather than kept from the count: IPT
  // ballots held across the barrier would not fit the scalar registers
  uint32_t thr_c = thr;
  asm volatile("" : "+s"(thr_c));
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const bool c = raw_at_least<POS>(b[i], thr_c);
    const uint64_t mk = __ballot(c);
    const uint32_t q = at + (uint32_t)lanes_below(mk);
    if (c && (POS || q < total)) {
      sm.cand[q] = b[i];
      sm.cidx[q] = (uint32_t)(base + 64 * i + lane);
    }
    at += (uint32_t)__popcll(mk);
  }
  __syncthreads(); // the candidates are complete (and red is read)
  // the sample's largest key bounds the first pass's bins, which need no
  // per-score maximum: the row's keys above it share the top bin
  select_compacted<NT>(sm, (int)total, thr, smax > thr ? smax : thr, k, ib, out);
  return true;
}

// Selects the top k of a row of E > k scores, IPT keys per lane.
template <int NT, int IPT>
__device__ __forceinline__ void select_row(const float *row, int E, int k, int32_t *out,
                                           int32_t ib, TopkShared &sm) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // Wave w holds row indices [w * IPT * 64, (w + 1) * IPT * 64): item i of a
  // lane is index base + 64 i + lane, so every slot past the row is an index
  // >= E, after every index of the row in item order.
  const int base = wave * IPT * 64;

  // Loads through a buffer resource bounded by the row's E scores: past the
  // row they return 0 without a predicate and touch no memory; such items
  // get key 0 when keys are formed (every visible key is > 0x007FFFFF). The
  // item step is part of the vector offset, which the hardware checks against
  // the bound (the scalar offset is not checked).
  const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(row), (short)0, E * 4, 0x00020000);
  // ---- the sample for the threshold estimate goes out first: 16 consecutive
  // scores out of every 256 (a sixteenth of the row's bytes), so that the
  // estimate runs while the row's own loads are still arriving (one CU pulls
  // a row at ~28 GB/s: ~5 us for 32K scores).
  constexpr int SPT = (IPT + 15) / 16; // sampled scores per lane (E <= IPT * NT)
  uint32_t sbits[SPT];
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    const int q = tid + NT * u;
    sbits[u] = __builtin_amdgcn_raw_buffer_load_b32(rr, (uint32_t)((q >> 4) * 256 + (q & 15)) * 4u, 0, 0);
  }
  uint32_t key[IPT]; // the row's raw bits; keys only on the full passes
  const uint32_t voff = (uint32_t)(base + lane) * 4u;
  const int left = E - base - lane; // item i is visible iff 64 * i < left
#pragma unroll
  for (int i = 0; i < IPT; ++i) key[i] = __builtin_amdgcn_raw_buffer_load_b32(rr, voff + 256u * i, 0, 0);
  if (tid == 0) {
    sm.ncand = 0;
    sm.nsmall = 0;
  }
  // the histogram starts zeroed (ordered before the first pass by the
  // barrier of block_max_min)
#pragma unroll
  for (int q = 0; q < kBins / NT; ++q) sm.hist[tid * (kBins / NT) + q] = 0u;

  // ---- sampled threshold: the lower edge thr0 of the value bin (linear
  // between the sample's extremes) that holds the m-th largest of the n_smp
  // sampled keys, m chosen so that about min(2k, (k + kCandCap) / 2) of the
  // row's keys lie at or above it. When between k and kCandCap of them do
  // (counted exactly), those keys and their indices are compacted into LDS
  // in index order, and the exact selection and the output run over them
  // alone. Otherwise the estimate is dropped (nothing is decided by it) and
  // the full passes over the row follow.
  const bool sampled = E > kCandCap && 2 * k <= kCandCap;
  uint32_t thr0 = 0u, smax0 = 0u; // the estimate and the sample's largest key
  bool estimated = false;
  if (sampled) {
    uint32_t smp[SPT], smax = 0u, smin = 0xFFFFFFFFu, n_smp = 0u;
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const int q = tid + NT * u;
      smp[u] = (q >> 4) * 256 + (q & 15) < E ? float_key(__uint_as_float(sbits[u])) : 0u;
      if (smp[u] != 0u) {
        smax = smp[u] > smax ? smp[u] : smax;
        smin = smp[u] < smin ? smp[u] : smin;
      }
      n_smp += (uint32_t)__popcll(__ballot(smp[u] != 0u));
    }
    block_max_min<NT>(sm, smax, smin, n_smp); // n_smp > 0: position 0 is sampled
    const float h0 = key_float(smin) * 0.5f;
    const float hr = key_float(smax) * 0.5f - h0;
    const float scale = (float)kBins / hr;
    if (hr > 0.f && scale < 3.0e38f) {
      auto vbin = [&](uint32_t kk) -> uint32_t {
        const float x = __builtin_fmaf(key_float(kk), 0.5f, -h0) * scale;
        return (uint32_t)fminf(x, (float)(kBins - 1));
      };
      const int target = (k + kCandCap) / 2 < 2 * k ? (k + kCandCap) / 2 : 2 * k;
      const int64_t mm = ((int64_t)n_smp * target + E - 1) / E;
      const int m = mm < 1 ? 1 : (mm > (int64_t)n_smp ? (int)n_smp : (int)mm);
      uint32_t b0;
      int a0, i0;
      radix_pass<NT>(
          sm, m,
          [&](auto add) {
#pragma unroll
            for (int u = 0; u < SPT; ++u)
              if (smp[u] != 0u) add(vbin(smp[u]));
          },
          b0, a0, i0);
      thr0 = first_key_in_bin_near(smin - 1u, smax, b0, bin_edge_key(b0, h0, scale), vbin);
      smax0 = smax;
      estimated = true;
    }
  }
  if (estimated) {
    // Counted and compacted on the raw bits, one compare per score, with no
    // key formed: per score this phase is bound by vector-ALU issue (16 waves
    // x IPT scores per CU), and only the candidates are keyed, as they are
    // read. A threshold at exactly +0's key moves to the key below it, which
    // no score has (-0 keys as +0): the same scores pass, and the threshold
    // then lies strictly above or below +0's key.
    if (thr0 == 0x80000000u) thr0 = 0x7FFFFFFFu;
    // red was last read (block_max_min) before radix_pass's barriers
    if (thr0 > 0x80000000u ? count_compact<NT, IPT, true>(sm, key, thr0, smax0, E, k, base, ib, out)
                           : count_compact<NT, IPT, false>(sm, key, thr0, smax0, E, k, base, ib, out))
      return;
  }
  // keys for the full passes
#pragma unroll
  for (int i = 0; i < IPT; ++i) key[i] = 64 * i < left ? float_key(__uint_as_float(key[i])) : 0u;

  // ---- the row's extremes, for the full passes
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu, unused = 0u;
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    if (key[i] != 0u) {
      kmax = key[i] > kmax ? key[i] : kmax;
      kmin = key[i] < kmin ? key[i] : kmin;
    }
  }
  if (sampled) __syncthreads(); // red was read above
  block_max_min<NT>(sm, kmax, kmin, unused);

  // The candidates are the keys in [lo, hi]; `need` of them remain to take.
  uint32_t lo = kmin, hi = kmax;
  int need = k, cand = E;
  uint32_t thr;    // final rule: key > thr, plus need_eq keys == thr (lowest index first)
  int need_eq = 0; // 0: every key >= thr + 1 is taken
  int n_eq_total = -1;
  bool done = false;
  bool in_lds = false; // the candidates are sm.cand[0, nc)
  int nc = 0;

  // Bins by value, linear between the row's extremes (a monotone map: a
  // higher bin holds only larger scores; halved so nothing overflows).
  const float h0 = key_float(kmin) * 0.5f;
  const float hr = key_float(kmax) * 0.5f - h0;
  const float scale = (float)kBins / hr;
  const bool linear = hr > 0.f && scale < 3.0e38f;
  // one explicit FMA, so every evaluation of a key's bin rounds alike
  auto vbin = [&](uint32_t kk) -> uint32_t {
    const float x = __builtin_fmaf(key_float(kk), 0.5f, -h0) * scale;
    return (uint32_t)fminf(x, (float)(kBins - 1));
  };

  // ---- pass 1 over every key, by value bin
  if (linear) {
    uint32_t bin;
    int above, inbin;
    radix_pass<NT>(
        sm, need,
        [&](auto add) {
#pragma unroll
          for (int i = 0; i < IPT; ++i)
            if (key[i] != 0u) add(vbin(key[i]));
        },
        bin, above, inbin);
    need -= above;
    cand = inbin;
    // The bin's keys form one key interval [lo, hi] (the bin is monotone in
    // the key); every wave finds its ends from the uniform kmin, kmax and bin
    // alike, so no pass over the keys and no barrier. The bin is not empty,
    // so its first key is <= kmax and has bin exactly `bin`.
    lo = first_key_in_bin_near(kmin - 1u, kmax, bin, bin_edge_key(bin, h0, scale), vbin);
    hi = bin + 1 < (uint32_t)kBins && vbin(kmax) > bin
             ? first_key_in_bin_near(lo, kmax, bin + 1, bin_edge_key(bin + 1, h0, scale), vbin) - 1u
             : kmax;
    if (inbin == need) {
      thr = lo - 1u; // lo >= kmin > 0
      done = true;
    }
  }

  // ---- then by key bits within [lo, hi], over the candidates compacted into
  // LDS when they fit, else over the registers
  if (!done && !in_lds && cand > kRankCap && cand <= kCandCap) {
    in_lds = true;
    nc = cand;
    // the wave's candidates are counted from ballots first, so the wave
    // reserves its slots with one LDS atomic instead of one per item
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < IPT; ++i) mine += key[i] >= lo && key[i] <= hi ? 1u : 0u;
    const uint32_t tot = wave_sum(mine);
    uint32_t at = 0;
    if (lane == 0 && tot != 0u) at = atomicAdd(&sm.ncand, tot);
    at = __builtin_amdgcn_readlane(at, 0);
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const bool c = key[i] >= lo && key[i] <= hi;
      const uint64_t m = __ballot(c);
      if (c) sm.cand[at + lanes_below(m)] = key[i];
      at += (uint32_t)__popcll(m);
    }
    __syncthreads();
  }
  while (!done) {
    if (lo == hi) { // a single key value
      thr = lo;
      need_eq = need;
      n_eq_total = cand;
      break;
    }
    if (cand <= kRankCap) {
      // one wave ranks the candidates: compact them, lane l holds candidate l
      auto put = [&](uint32_t x, bool c) {
        const uint64_t m = __ballot(c);
        if (m) {
          uint32_t at = 0;
          if (lane == 0) at = atomicAdd(&sm.nsmall, (uint32_t)__popcll(m));
          at = __builtin_amdgcn_readlane(at, 0);
          if (c) sm.small[at + lanes_below(m)] = x;
        }
      };
      const bool direct = in_lds && cand == nc; // every compacted key is a candidate
      if (direct) {
        // sm.cand is complete since the barrier after the compaction
      } else if (in_lds) {
        for (int c0 = wave * 64; c0 < nc; c0 += NT) {
          const int c = c0 + lane;
          const uint32_t x = c < nc ? sm.cand[c] : 0u;
          put(x, c < nc && x >= lo && x <= hi);
        }
        __syncthreads();
      } else {
        // from the registers: count, one reservation per wave, then write
        uint32_t mine = 0;
#pragma unroll
        for (int i = 0; i < IPT; ++i) mine += key[i] >= lo && key[i] <= hi ? 1u : 0u;
        const uint32_t tot = wave_sum(mine);
        uint32_t at = 0;
        if (lane == 0 && tot != 0u) at = atomicAdd(&sm.nsmall, tot);
        at = __builtin_amdgcn_readlane(at, 0);
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
          const bool c = key[i] >= lo && key[i] <= hi;
          const uint64_t m = __ballot(c);
          if (c) sm.small[at + lanes_below(m)] = key[i];
          at += (uint32_t)__popcll(m);
        }
        __syncthreads();
      }
      if (wave == 0) {
        const uint32_t *src = direct ? sm.cand : sm.small;
        const uint32_t mykey = lane < cand ? src[lane] : 0u;
        int gt = 0, eq = 0;
        for (int j = 0; j < cand; ++j) {
          const uint32_t x = __builtin_amdgcn_readlane(mykey, j);
          gt += x > mykey ? 1 : 0;
          eq += x == mykey ? 1 : 0;
        }
        const bool is_thr = lane < cand && gt < need && gt + eq >= need;
        const int tl = (int)__builtin_ctzll(__ballot(is_thr));
        if (lane == tl) {
          sm.sel[0] = mykey;
          sm.sel[1] = (uint32_t)(need - gt);
          sm.sel[2] = (uint32_t)eq;
        }
      }
      __syncthreads();
      thr = sm.sel[0];
      need_eq = (int)sm.sel[1];
      n_eq_total = (int)sm.sel[2];
      break;
    }
    const uint32_t range = hi - lo;
    const int bits = 32 - __builtin_clz(range);
    const int shift = bits > kDigitBits ? bits - kDigitBits : 0;
    uint32_t bin;
    int above, inbin;
    if (in_lds) {
      radix_pass<NT>(
          sm, need,
          [&](auto add) {
            for (int c = tid; c < nc; c += NT) {
              const uint32_t x = sm.cand[c];
              if (x >= lo && x <= hi) add((x - lo) >> shift);
            }
          },
          bin, above, inbin);
    } else {
      radix_pass<NT>(
          sm, need,
          [&](auto add) {
#pragma unroll
            for (int i = 0; i < IPT; ++i)
              if (key[i] >= lo && key[i] <= hi) add((key[i] - lo) >> shift);
          },
          bin, above, inbin);
    }
    need -= above;
    cand = inbin;
    const uint32_t nlo = lo + (bin << shift);
    const uint32_t width = (1u << shift) - 1u;
    hi = hi - nlo < width ? hi : nlo + width;
    lo = nlo;
    if (inbin == need) { // the whole bin is taken
      thr = lo - 1u;
      break;
    }
  }
  // every key equal to thr is taken: the rule is key >= thr_ge
  const bool all_ties = need_eq == 0 || need_eq == n_eq_total;
  const uint32_t thr_ge = need_eq == 0 ? thr + 1u : thr;

  emit_selection<NT, IPT>(
      sm, [&](int i) -> uint32_t { return key[i]; },
      [&](int i) -> int32_t { return ib + base + i * 64 + lane; }, thr, need_eq, all_ties, thr_ge,
      k, out);
}

template <int NT, int MAXIPT>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
  __shared__ TopkShared sm;
  const int tid = threadIdx.x;
  if (tid < 3) sm.sel[tid] = 0; // read only after barriers that follow this
  const int r = blockIdx.x;
  const int b = r / a.next_n;
  const int j = r - b * a.next_n;
  int64_t E64 = (int64_t)a.lens[b] - (a.next_n - 1 - j);
  if (E64 < 0) E64 = 0;
  if (E64 > a.W) E64 = a.W;
  const int E = (int)E64;
  const int k = a.k;
  int32_t *out = a.out_idx + (int64_t)r * k;
  if (a.out_count && tid == 0) a.out_count[r] = E < k ? E : k;

  if (E <= k) { // everything visible is selected
    for (int i = tid; i < k; i += NT) out[i] = i < E ? a.index_base + i : -1;
    return;
  }
  const float *row = a.logits + (int64_t)r * a.W;
  // the smallest bucket of keys per lane that holds the row
  const int32_t ib = a.index_base;
  if (E <= NT * 4) select_row<NT, 4>(row, E, k, out, ib, sm);
  else if (MAXIPT >= 8 && E <= NT * 8) select_row<NT, (MAXIPT >= 8 ? 8 : 4)>(row, E, k, out, ib, sm);
  else if (MAXIPT >= 16 && E <= NT * 16)
    select_row<NT, (MAXIPT >= 16 ? 16 : 4)>(row, E, k, out, ib, sm);
  else if (MAXIPT >= 32 && E <= NT * 32)
    select_row<NT, (MAXIPT >= 32 ? 32 : 4)>(row, E, k, out, ib, sm);
  else if (MAXIPT >= 64) select_row<NT, (MAXIPT >= 64 ? 64 : 4)>(row, E, k, out, ib, sm);
}


// ---- one wave per row, for widths up to 4096 --------------------------------
//
// Short rows (prefill widths) are cheap enough that work-group barriers would
// dominate, so each wave owns a whole row: its keys (up to 64 per lane) stay in
// registers and the radix select runs on a per-wave LDS histogram with no
// barrier at all. The first pass bins the row by score value, linearly between
// the row's minimum and maximum: the map is monotone (every step rounds
// monotonically), so a higher bin holds only larger scores, and scores spread
// over the bins far more evenly than their float bit patterns would. The
// chosen bin's keys, between its smallest and largest key, are then either
// ranked directly (at most 64 of them) or binned again by key bits.

constexpr int kWaveBins = 1024;
constexpr int kRowsPerGroup = 4; // waves (rows) per work group
constexpr int kWaveCand = 64;

struct WaveShared {
  uint32_t hist[kWaveBins];
  uint32_t cand[kWaveCand];
};

// Waits for this wave's LDS operations; a wave's LDS accesses are then
// visible to its own later reads in every lane.
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0); vmcnt / expcnt not waited
  __builtin_amdgcn_wave_barrier();
}

// Histogram of the keys accepted by `bin_of` (which returns kWaveBins for a
// key it skips), then the bin holding the need-th largest: its index, the
// count in higher bins and the count in it, uniform over the wave.
template <int IPT, typename BinOf>
__device__ __forceinline__ void wave_radix_pass(WaveShared &sm, const uint32_t (&key)[IPT], int need,
                                                BinOf bin_of, uint32_t &bin, int &above,
                                                int &inbin) {
  const int lane = threadIdx.x & 63;
  uint4 *h4 = reinterpret_cast<uint4 *>(sm.hist);
#pragma unroll
  for (int q = 0; q < kWaveBins / 256; ++q) h4[q * 64 + lane] = uint4{0u, 0u, 0u, 0u};
  wave_lds_sync();
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const uint32_t d = bin_of(key[i]);
    if (d < (uint32_t)kWaveBins) atomicAdd(&sm.hist[d], 1u);
  }
  wave_lds_sync();
  // lane l scans bins [kWaveBins - 16 (l + 1), kWaveBins - 16 l) from the top
  const uint4 *r4 = reinterpret_cast<const uint4 *>(sm.hist + kWaveBins - 16 * (lane + 1));
  uint32_t cnt[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = r4[q];
    cnt[4 * q] = v.x;
    cnt[4 * q + 1] = v.y;
    cnt[4 * q + 2] = v.z;
    cnt[4 * q + 3] = v.w;
  }
  uint32_t mine = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) mine += cnt[q];
  const uint32_t incl = wave_incl_scan_u32(mine);
  const uint32_t excl = incl - mine;
  const bool holder = excl < (uint32_t)need && incl >= (uint32_t)need;
  uint32_t my_bin = 0, my_above = 0, my_in = 0;
  if (holder) {
    uint32_t run = excl;
#pragma unroll
    for (int q = 15; q >= 0; --q) { // the lane's highest bin first
      if (run < (uint32_t)need && run + cnt[q] >= (uint32_t)need) {
        my_bin = (uint32_t)(kWaveBins - 16 * (lane + 1) + q);
        my_above = run;
        my_in = cnt[q];
      }
      run += cnt[q];
    }
  }
  // exactly one lane holds the need-th key: the counted keys number >= need
  const int hl = (int)__builtin_ctzll(__ballot(holder));
  bin = __builtin_amdgcn_readlane(my_bin, hl);
  above = (int)__builtin_amdgcn_readlane(my_above, hl);
  inbin = (int)__builtin_amdgcn_readlane(my_in, hl);
}

template <int IPT>
__device__ __forceinline__ void select_row_wave(const float *row, int E, int k, int32_t *out,
                                                int32_t ib, WaveShared &sm) {
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(row), (short)0, E * 4, 0x00020000);
  uint32_t key[IPT]; // item i holds index 64 i + lane; 0 past the row
  const int left = E - lane;
#pragma unroll
  for (int i = 0; i < IPT; ++i) { // bounded like the block kernel's loads
    const uint32_t bits =
        __builtin_amdgcn_raw_buffer_load_b32(rr, (uint32_t)lane * 4u + 256u * i, 0, 0);
    key[i] = 64 * i < left ? float_key(__uint_as_float(bits)) : 0u;
  }
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    if (key[i] != 0u) {
      kmax = key[i] > kmax ? key[i] : kmax;
      kmin = key[i] < kmin ? key[i] : kmin;
    }
  }
  kmax = wave_max_u32(kmax);
  kmin = wave_min_u32(kmin);

  // The candidates are the keys in [lo, hi]; `need` of them remain to take.
  uint32_t lo = kmin, hi = kmax;
  int need = k, cand = E;
  uint32_t thr;    // final rule: key > thr, plus need_eq keys == thr (lowest index first)
  int need_eq = 0; // 0: every key >= thr + 1 is taken
  int n_eq_total = -1;
  bool done = false;

  // ---- pass 1 by value, linear between the row's extremes (halved so the
  // difference cannot overflow)
  const float h0 = key_float(kmin) * 0.5f;
  const float hr = key_float(kmax) * 0.5f - h0;
  const float scale = (float)kWaveBins / hr;
  if (hr > 0.f && scale < 3.0e38f) {
    // one explicit FMA, so every evaluation of a key's bin rounds alike
    auto vbin = [&](uint32_t kk) -> uint32_t {
      const float x = __builtin_fmaf(key_float(kk), 0.5f, -h0) * scale;
      return (uint32_t)fminf(x, (float)(kWaveBins - 1));
    };
    uint32_t bin;
    int above, inbin;
    wave_radix_pass<IPT>(
        sm, key, need, [&](uint32_t kk) { return kk != 0u ? vbin(kk) : (uint32_t)kWaveBins; }, bin,
        above, inbin);
    need -= above;
    cand = inbin;
    // the bin's keys form the key interval [lo, hi] (see the block kernel)
    lo = first_key_in_bin_near(kmin - 1u, kmax, bin, bin_edge_key(bin, h0, scale), vbin);
    hi = bin + 1 < (uint32_t)kWaveBins && vbin(kmax) > bin
             ? first_key_in_bin_near(lo, kmax, bin + 1, bin_edge_key(bin + 1, h0, scale), vbin) - 1u
             : kmax;
    if (inbin == need) {
      thr = lo - 1u; // lo >= kmin > 0
      done = true;
    }
  }
  // ---- then by key bits within [lo, hi]
  while (!done) {
    if (lo == hi) { // a single key value
      thr = lo;
      need_eq = need;
      n_eq_total = cand;
      break;
    }
    if (cand <= kWaveCand) {
      // rank the candidates directly: lane l holds candidate l
      uint32_t at = 0;
#pragma unroll
      for (int i = 0; i < IPT; ++i) {
        const bool c = key[i] >= lo && key[i] <= hi;
        const uint64_t m = __ballot(c);
        if (c) sm.cand[at + lanes_below(m)] = key[i];
        at += (uint32_t)__popcll(m);
      }
      wave_lds_sync();
      const uint32_t mykey = lane < cand ? sm.cand[lane] : 0u;
      int gt = 0, eq = 0;
      for (int j = 0; j < cand; ++j) {
        const uint32_t x = __builtin_amdgcn_readlane(mykey, j);
        gt += x > mykey ? 1 : 0;
        eq += x == mykey ? 1 : 0;
      }
      const bool is_thr = lane < cand && gt < need && gt + eq >= need;
      const int tl = (int)__builtin_ctzll(__ballot(is_thr));
      thr = __builtin_amdgcn_readlane(mykey, tl);
      n_eq_total = __builtin_amdgcn_readlane(eq, tl);
      need_eq = need - __builtin_amdgcn_readlane(gt, tl);
      break;
    }
    const uint32_t range = hi - lo;
    const int bits = 32 - __builtin_clz(range);
    const int shift = bits > 10 ? bits - 10 : 0;
    uint32_t bin;
    int above, inbin;
    wave_radix_pass<IPT>(
        sm, key, need,
        [&](uint32_t kk) {
          return kk >= lo && kk <= hi ? (kk - lo) >> shift : (uint32_t)kWaveBins;
        },
        bin, above, inbin);
    need -= above;
    cand = inbin;
    const uint32_t nlo = lo + (bin << shift);
    const uint32_t width = (1u << shift) - 1u;
    hi = hi - nlo < width ? hi : nlo + width;
    lo = nlo;
    if (inbin == need) { // the whole bin is taken
      thr = lo - 1u;
      break;
    }
  }
  const bool all_ties = need_eq == 0 || need_eq == n_eq_total;
  const uint32_t thr_ge = need_eq == 0 ? thr + 1u : thr;

  // ---- indices in ascending order
  int pos = 0, eq_seen = 0;
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    bool sel;
    if (all_ties) {
      sel = key[i] >= thr_ge;
    } else {
      const bool eq = key[i] == thr;
      const uint64_t meq = __ballot(eq);
      sel = key[i] > thr || (eq && eq_seen + lanes_below(meq) < need_eq);
      eq_seen += (int)__popcll(meq);
    }
    const uint64_t msel = __ballot(sel);
    const int p = pos + lanes_below(msel);
    if (sel && p < k) out[p] = ib + 64 * i + lane;
    pos += (int)__popcll(msel);
  }
}

__global__ __launch_bounds__(64 * kRowsPerGroup) void topk_wave_kernel(TopkArgs a) {
  __shared__ WaveShared sm[kRowsPerGroup];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * kRowsPerGroup + wave;
  if (r >= a.R) return; // waves are independent: no work-group barrier below
  const int b = r / a.next_n;
  const int j = r - b * a.next_n;
  int64_t E64 = (int64_t)uniform_load(a.lens + b) - (a.next_n - 1 - j);
  if (E64 < 0) E64 = 0;
  if (E64 > a.W) E64 = a.W;
  const int E = (int)E64;
  const int k = a.k;
  int32_t *out = a.out_idx + (int64_t)r * k;
  if (a.out_count && lane == 0) a.out_count[r] = E < k ? E : k;
  if (E <= k) {
    for (int i = lane; i < k; i += 64) out[i] = i < E ? a.index_base + i : -1;
    return;
  }
  const float *row = a.logits + (int64_t)r * a.W;
  if (E <= 1024) select_row_wave<16>(row, E, k, out, a.index_base, sm[wave]);
  else if (E <= 2048) select_row_wave<32>(row, E, k, out, a.index_base, sm[wave]);
  else select_row_wave<64>(row, E, k, out, a.index_base, sm[wave]);
}

template <int NT, int MAXIPT> hipError_t launch_rows(const TopkArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((topk_kernel<NT, MAXIPT>), dim3(a.R), dim3(NT), 0, s, a);
  return hipGetLastError();
}

} // namespace

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
  // one wave per row pays off once there are rows enough to fill the chip; a
  // few short rows (a single decode sequence, a prefill tail chunk) finish
  // sooner with a whole work group each
  if (a.W <= 4096 && a.R >= 2048) {
    const int groups = (a.R + kRowsPerGroup - 1) / kRowsPerGroup;
    hipLaunchKernelGGL(topk_wave_kernel, dim3(groups), dim3(64 * kRowsPerGroup), 0, s, a);
    return hipGetLastError();
  }
  return launch_rows<1024, 64>(a, s);
}

} // namespace idx
