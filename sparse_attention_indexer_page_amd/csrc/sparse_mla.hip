// Sparse attention over the indexer's selection on gfx950: every query row
// attends to its own top-k tokens only (flashinfer PR #3269 "Add DeepSeek V4
// sparse MLA TRTLLM-GEN kernels": a decode over dynamic per-row top-k lengths
// with 512-dim QK and V; in MLA the values are the same latent rows as the
// keys). For row r (sequence b = r / next_n), head h and the n_r =
// min(topk_lens[r], k) listed tokens t_i (entries < 0 skipped):
//     s_i = scale * (q[r][h] . c[t_i]),   out[r][h] = sum_i softmax(s)_i c[t_i]
// with c[t] the bf16 latent row of token t through the block table.
//
// Split over tokens (flash decoding): work group (split, r) = 8 waves, wave w
// owning heads 16 (w & 3) .. + 15 and output dims 256 (w >> 2) .. + 255,
// scores a contiguous chunk of row r's list in blocks of 32 tokens:
//   * a prologue resolves every listed token of the chunk through the block
//     table once and keeps the byte offsets of their latent rows in LDS; the
//     wave's 16 query heads (its 256 dims of them) stay in VGPRs as MFMA B
//     operands;
//   * the rows of a block (32 KB; thread t loads 64 bytes of row t / 16) are
//     loaded into registers four blocks ahead of the one being scored (three
//     blocks, 96 KB per work group, stay in flight at every wait), then
//     written into one of two LDS slots (rows padded to 1040 bytes); a
//     skipped entry reads a fixed in-bounds row and is stored as zeros.
//     (Direct-to-LDS loads would save the register hop, but the compiler then
//     waits for every one in flight before any LDS read of the slots.)
//   * S^T = K q^T on v_mfma_f32_16x16x32_bf16 (tokens x heads, two 16-token
//     tiles): the two waves of a head group each take 8 of the 16 k-steps
//     (256 dims) and swap their partial tiles through LDS, both summing them
//     in the same order, so both hold the same scores;
//   * online softmax per head over the block; the scores come out of that
//     MFMA in the A-operand layout of the P.V product (lane l: head l & 15,
//     k-slots 8g..8g+7 = tokens 4g..4g+3 of both tiles), so P needs no
//     shuffle, only its split into a bf16 part and a bf16 remainder;
//   * O += P V on v_mfma_f32_16x16x32_bf16 (heads x 16 dims, K = the 32
//     tokens), two products per tile (the two parts of P), 16 tiles for the
//     wave's 256 dims, fp32 accumulators in VGPRs;
//     a lane reads 8-byte runs of 4 dims per token and byte-permutes them
//     into the token-major B operands of 4 tiles (a tile's 16 columns are
//     then every fourth dim), rather than reading 2-byte columns.
// Each chunk leaves (max, sum, unnormalized O) per head in the workspace; a
// second launch merges the chunks of every (row, head) and writes bf16 out
// and the log-sum-exp.
#include "device_common.h"
#include "internal.h"

namespace idx {
namespace {

using namespace dev;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kMlaHeads = 64;
constexpr int kMlaDim = 512;
constexpr int kBlk = 32;                   // tokens per block (two 16-token tiles)
constexpr int kTileRow = 2 * kMlaDim + 16; // LDS bytes per staged row
constexpr int kAhead = 4;                  // blocks loaded ahead of the one being scored
constexpr int kThreads = 512;              // 4 head groups x 2 dim halves
constexpr int kWaveDims = kMlaDim / 2;     // output dims per wave

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ inline uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Work-group barrier that waits for the wave's LDS operations only: a
// __syncthreads would also wait for the loads of the blocks ahead.
__device__ inline void lds_only_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48) with the gfx950 row swaps: no LDS round trip, and every lane adds
// the same operands in the same order.
__device__ inline float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

struct MlaState {
  v8bf qb[kWaveDims / 32]; // head col of the wave's group, dims 256 dh + 32 kk + 8 g .. + 8
  v4f O[kWaveDims / 16]; // heads 4g + jj; tile 4 p + j: dims 64 p + 4 col + j of the wave's half
  float m_run, l_run;    // head col of the wave's group
};

// Token of P.V k-slot 8 g + i: slots 0..3 of lane group g are tile 0's
// tokens 4g..4g+3, slots 4..7 tile 1's (16 + 4g ..), which is where the
// score MFMAs leave them, so P needs no shuffle.
__device__ inline int pv_token(int g, int i) { return i < 4 ? 4 * g + i : 16 + 4 * g + (i - 4); }

// Scores one block from its LDS slot (all 32 rows resident); dh: the wave's
// dim half; xch: the work group's exchange area for partial score tiles
// (two v4f per lane and wave).
__device__ inline void score_block(const MlaArgs &a, MlaState &S, const uint8_t *tile, int dh,
                                   v4f *xch, const int64_t *row_off_blk) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int col = lane & 15;
  // ---- partial S^T = K q^T of both 16-token tiles over the wave's 256
  // dims: lane holds head col, tokens 16 tt + 4g..+3 (A: token col, B: head
  // col, both dims 256 dh + 32 kk + 8 g .. + 8); two independent chains
  v4f part[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const uint8_t *kt = tile + col * kTileRow + 2 * kWaveDims * dh + 16 * g;
#pragma unroll
  for (int kk = 0; kk < kWaveDims / 32; ++kk) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const v8bf ka = *reinterpret_cast<const v8bf *>(kt + 16 * tt * kTileRow + 64 * kk);
      part[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, S.qb[kk], part[tt], 0, 0, 0);
    }
    if ((kk & 1) == 1) __builtin_amdgcn_sched_barrier(0); // operands of four MFMAs at a time
  }
  // ---- the partner wave (other dim half, same heads) holds the other
  // half of the sums; both add dim half 0 + dim half 1
  xch[wave * 64 + lane] = part[0];
  xch[kThreads + wave * 64 + lane] = part[1];
  lds_only_barrier();
  float s[2][4];
  float bm = -__builtin_huge_valf();
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const v4f other = xch[tt * kThreads + (wave ^ 4) * 64 + lane];
    const v4f st = dh == 0 ? part[tt] + other : other + part[tt];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      s[tt][jj] = row_off_blk[16 * tt + 4 * g + jj] >= 0 ? st[jj] * a.scale : -__builtin_huge_valf();
      bm = fmaxf(bm, s[tt][jj]);
    }
  }
  // ---- online softmax over the block, per head
  bm = rows_max(bm);
  const float m_new = fmaxf(S.m_run, bm);
  const float alpha = S.m_run == -__builtin_huge_valf() ? 0.f : __expf(S.m_run - m_new);
  float p[2][4], ls = 0.f;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      p[tt][jj] = s[tt][jj] == -__builtin_huge_valf() ? 0.f : __expf(s[tt][jj] - m_new);
      ls += p[tt][jj];
    }
  ls = rows_sum(ls);
  S.l_run = S.l_run * alpha + ls;
  S.m_run = m_new;
  // O rows are heads 4g + jj: their factors live in lanes 4g + jj
  float ah[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) ah[jj] = __shfl(alpha, 4 * g + jj, 64);
  // P as the A operand of the 16x16x32 product: head col, k-slots 8g..8g+7.
  // Each probability is split into its bf16 rounding and the bf16 rounding
  // of the remainder, and both parts multiply V: together they carry p to
  // about 2^-16 relative instead of bf16's 2^-8, so the output's only
  // sizeable error is its own final bf16 rounding.
  v8bf pa, pl;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float pv = p[i >> 2][i & 3];
    const uint32_t h = bf16_rne(pv);
    pa[i] = __builtin_bit_cast(__bf16, (uint16_t)h);
    pl[i] = __builtin_bit_cast(__bf16, (uint16_t)bf16_rne(pv - __uint_as_float(h << 16)));
  }
  // V operands: lane col reads 8 bytes (dims 4 col .. + 3 of a 64-dim
  // span) of each of its 8 tokens and regroups them into the B operands of
  // four tiles, tile j taking dim 4 col + j of every token (two tokens per
  // dword, by byte permutes)
  const uint8_t *tv = tile + 2 * kWaveDims * dh + 8 * col;
#pragma unroll
  for (int p4 = 0; p4 < kWaveDims / 64; ++p4) {
    uint2 w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i] = *reinterpret_cast<const uint2 *>(tv + pv_token(g, i) * kTileRow + 128 * p4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      v4i vb;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t lo = (j & 2) ? w[2 * m].y : w[2 * m].x;
        const uint32_t hi = (j & 2) ? w[2 * m + 1].y : w[2 * m + 1].x;
        vb[m] = (int)__builtin_amdgcn_perm(hi, lo, sel);
      }
      v4f &o = S.O[4 * p4 + j];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) o[jj] *= ah[jj];
      o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(v8bf, vb), o, 0, 0, 0);
      o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, __builtin_bit_cast(v8bf, vb), o, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0); // the V reads of one 64-dim span in flight
  }
}

__global__ __launch_bounds__(kThreads) void sparse_mla_partial_kernel(MlaArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kBlk * kTileRow];
  // byte offset of each listed row (-1: skipped, or past the chunk, up to
  // the last block loaded ahead)
  __shared__ int64_t row_off[kMlaMaxChunk + 2 * kAhead * kBlk];
  const int sp = blockIdx.x;
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave & 3; // head group
  const int dh = wave >> 2; // dim half
  const int g = lane >> 4;
  const int col = lane & 15;
  __shared__ v4f xch[2 * kThreads]; // partial score tiles, two per lane
  const int b = r / a.next_n;
  int n = uniform_load(a.topk_lens + r);
  n = n < 0 ? 0 : (n > a.k ? a.k : n);
  const int c0 = sp * a.chunk;
  const int c1 = c0 + a.chunk < n ? c0 + a.chunk : n;
  // blocks, rounded up to whole loop passes of kAhead: a block of skipped
  // rows leaves the softmax state exactly as it was
  int nblk = c1 > c0 ? (c1 - c0 + kBlk - 1) / kBlk : 0;
  nblk = (nblk + kAhead - 1) / kAhead * kAhead;

  // ---- the chunk's row offsets
  for (int i = tid; i < (nblk + kAhead) * kBlk; i += kThreads) {
    int64_t off = -1;
    const int c = c0 + i;
    if (c < c1) {
      const int t = a.indices[(int64_t)r * a.k + c];
      if (t >= 0) {
        const int64_t lp = t >> a.page_shift;
        if (lp < a.bt_stride) {
          const int64_t pg = a.block_tables[(int64_t)b * a.bt_stride + lp];
          if (pg >= 0 && pg < a.num_pages)
            off = pg * a.page_stride + (int64_t)(t & (a.page_size - 1)) * a.row_stride;
        }
      }
    }
    row_off[i] = off;
  }
  MlaState S;
  const uint16_t *qh = a.q + ((int64_t)r * kMlaHeads + 16 * hg + col) * kMlaDim + kWaveDims * dh;
#pragma unroll
  for (int kk = 0; kk < kWaveDims / 32; ++kk)
    S.qb[kk] = *reinterpret_cast<const v8bf *>(qh + 32 * kk + 8 * g);
#pragma unroll
  for (int dt = 0; dt < kWaveDims / 16; ++dt) S.O[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  S.m_run = -__builtin_huge_valf();
  S.l_run = 0.f;
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); // the queries, before any block load is counted
  __syncthreads();                           // the table is complete

  // thread t carries bytes [256 u + 16 (t & 15), + 16), u = 0..3, of row
  // t >> 4 of a block (each load instruction reads 256 contiguous bytes of
  // four rows)
  const int gj = tid >> 4;
  const int gs = tid & 15;
  // Loads of block bi; rows past the chunk (and skipped entries) read the
  // cache's first row, inside every valid cache, and are zeroed when stored,
  // so every path keeps the same loads in flight.
  auto load_block = [&](int bi, v4i (&v)[4]) {
    const int64_t off = row_off[bi * kBlk + gj];
    const v4i *src = reinterpret_cast<const v4i *>(a.kv + (off >= 0 ? off : 0) + 16 * gs);
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = src[16 * u];
  };
  auto store_block = [&](int bi, const v4i (&v)[4]) {
    const bool ok = row_off[bi * kBlk + gj] >= 0;
    v4i *dst = reinterpret_cast<v4i *>(tile[bi & 1] + gj * kTileRow + 16 * gs);
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[16 * u] = ok ? v[u] : v4i{0, 0, 0, 0};
  };
  // One block: store it (its slot was last read two blocks ago, before the
  // previous barrier), publish it, refill its registers kAhead blocks ahead
  // and score it. The exchange area is rewritten only after the next
  // block's first barrier, which every wave reaches after reading it.
  auto step = [&](int bi, v4i (&v)[4]) {
    store_block(bi, v);
    lds_only_barrier();
    load_block(bi + kAhead, v);
    score_block(a, S, tile[bi & 1], dh, xch, row_off + bi * kBlk);
  };

  v4i rg[kAhead][4]; // register ring: block bi lives in rg[bi % kAhead]
  if (nblk > 0) {
#pragma unroll
    for (int u = 0; u < kAhead; ++u) load_block(u, rg[u]);
    for (int bi = 0; bi < nblk; bi += kAhead) {
#pragma unroll
      for (int u = 0; u < kAhead; ++u) step(bi + u, rg[u]);
    }
  }

  // ---- this chunk's (max, sum, unnormalized O) per head
  const int64_t base = ((int64_t)r * a.nsplit + sp) * kMlaHeads + 16 * hg;
  // tile 4 p + j holds dims 64 p + 4 col + j of the wave's half
#pragma unroll
  for (int p4 = 0; p4 < kWaveDims / 64; ++p4)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      *reinterpret_cast<v4f *>(a.ws_o + (base + 4 * g + jj) * kMlaDim + kWaveDims * dh + 64 * p4 +
                               4 * col) =
          v4f{S.O[4 * p4][jj], S.O[4 * p4 + 1][jj], S.O[4 * p4 + 2][jj], S.O[4 * p4 + 3][jj]};
  if (g == 0 && dh == 0) {
    a.ws_ml[(base + col) * 2] = S.m_run;
    a.ws_ml[(base + col) * 2 + 1] = S.l_run;
  }
}

// Merge of the chunks of one (row, head): work group (head, row), 128
// threads x 4 dims.
__global__ __launch_bounds__(128) void sparse_mla_merge_kernel(MlaArgs a) {
  const int h = blockIdx.x;
  const int r = blockIdx.y;
  const int d0 = 4 * threadIdx.x;
  float M = -__builtin_huge_valf();
  for (int s = 0; s < a.nsplit; ++s)
    M = fmaxf(M, a.ws_ml[(((int64_t)r * a.nsplit + s) * kMlaHeads + h) * 2]);
  float L = 0.f;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  if (M != -__builtin_huge_valf()) {
    for (int s = 0; s < a.nsplit; ++s) {
      const int64_t row = ((int64_t)r * a.nsplit + s) * kMlaHeads + h;
      const float ms = a.ws_ml[row * 2];
      if (ms == -__builtin_huge_valf()) continue;
      const float w = __expf(ms - M);
      L += w * a.ws_ml[row * 2 + 1];
      const v4f v = *reinterpret_cast<const v4f *>(a.ws_o + row * kMlaDim + d0);
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] += w * v[j];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t *dst = a.out + ((int64_t)r * kMlaHeads + h) * kMlaDim + d0;
  const uint32_t lo = bf16_rne(o[0] * inv) | (bf16_rne(o[1] * inv) << 16);
  const uint32_t hi = bf16_rne(o[2] * inv) | (bf16_rne(o[3] * inv) << 16);
  *reinterpret_cast<uint2 *>(dst) = uint2{lo, hi};
  if (a.lse && threadIdx.x == 0)
    a.lse[(int64_t)r * kMlaHeads + h] = L > 0.f ? M + __logf(L) : -__builtin_huge_valf();
}

} // namespace

hipError_t launch_sparse_mla(const MlaArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(sparse_mla_partial_kernel, dim3(a.nsplit, a.R), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sparse_mla_merge_kernel, dim3(kMlaHeads, a.R), dim3(128), 0, s, a);
  return hipGetLastError();
}

} // namespace idx
