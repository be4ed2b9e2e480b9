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
// scores a contiguous chunk of row r's list in blocks of 16 tokens:
//   * a prologue resolves every listed token of the chunk through the block
//     table once and keeps the byte offsets of their latent rows in LDS; the
//     wave's 16 query heads stay in VGPRs as MFMA B operands;
//   * the rows of a block (16 KB; thread t loads 32 bytes of row t / 32) are
//     loaded into registers three blocks ahead of the one being scored, so
//     each work group keeps 48 KB of reads in flight, then written into one
//     of two LDS slots (rows padded to 1040 bytes so the four token rows one
//     P.V operand read touches fall in distinct banks); a skipped entry
//     reads a fixed in-bounds row and is stored as zeros. (Direct-to-LDS
//     loads would save the register hop, but the compiler then waits for
//     every one in flight before any LDS read of the ring.)
//   * S^T = K q^T on v_mfma_f32_16x16x32_bf16 (tokens x heads, 512 dims = 16
//     k-steps); both waves of a head group compute it, so each holds the
//     scores of its heads without an exchange;
//   * online softmax per head; the scores come out of that MFMA in exactly
//     the A-operand layout of the P.V product (lane l: head l & 15, tokens
//     4g..4g+3), so P needs no shuffle, only bf16 rounding;
//   * O += P V on v_mfma_f32_16x16x16_bf16 (heads x 16 dims, K = the 16
//     tokens), 16 tiles for the wave's 256 dims, fp32 accumulators in VGPRs.
// Each chunk leaves (max, sum, unnormalized O) per head in the workspace; a
// second launch merges the chunks of every (row, head) and writes bf16 out
// and the log-sum-exp.
#include "device_common.h"
#include "internal.h"

namespace idx {
namespace {

using namespace dev;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int kMlaHeads = 64;
constexpr int kMlaDim = 512;
constexpr int kBlk = 16;                   // tokens per block
constexpr int kTileRow = 2 * kMlaDim + 16; // LDS bytes per staged row
constexpr int kAhead = 3;                  // blocks loaded ahead of the one being scored
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

struct MlaState {
  v8bf qb[kMlaDim / 32]; // head col of the wave's group, dims 32 kk + 8 g .. + 8
  v4f O[kWaveDims / 16]; // heads 4g + jj, dims 16 dt + col of the wave's half
  float m_run, l_run;    // head col of the wave's group
};

// Scores one block from its LDS slot (all 16 rows resident); dh: the wave's
// dim half.
__device__ inline void score_block(const MlaArgs &a, MlaState &S, const uint8_t *tile, int dh,
                                   const int64_t *row_off_blk) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int col = lane & 15;
  // ---- S^T = K q^T: lane holds head col, tokens 4g..4g+3 (A: token col,
  // B: head col, both dims 32 kk + 8 g .. + 8)
  v4f st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < kMlaDim / 32; ++kk) {
    const v8bf ka = *reinterpret_cast<const v8bf *>(tile + col * kTileRow + 64 * kk + 16 * g);
    st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, S.qb[kk], st, 0, 0, 0);
    if ((kk & 3) == 3) __builtin_amdgcn_sched_barrier(0); // operands of four steps at a time
  }
  // ---- online softmax over the block, per head
  float s[4];
  float bm = -__builtin_huge_valf();
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    s[jj] = row_off_blk[4 * g + jj] >= 0 ? st[jj] * a.scale : -__builtin_huge_valf();
    bm = fmaxf(bm, s[jj]);
  }
  bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
  bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
  const float m_new = fmaxf(S.m_run, bm);
  const float alpha = S.m_run == -__builtin_huge_valf() ? 0.f : __expf(S.m_run - m_new);
  float p[4], ls = 0.f;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    p[jj] = s[jj] == -__builtin_huge_valf() ? 0.f : __expf(s[jj] - m_new);
    ls += p[jj];
  }
  ls += __shfl_xor(ls, 16, 64);
  ls += __shfl_xor(ls, 32, 64);
  S.l_run = S.l_run * alpha + ls;
  S.m_run = m_new;
  // O rows are heads 4g + jj: their factors live in lanes 4g + jj
  float ah[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) ah[jj] = __shfl(alpha, 4 * g + jj, 64);
  // P as the A operand: head col, tokens 4g..4g+3, bf16
  const v4s pa = v4s{(short)bf16_rne(p[0]), (short)bf16_rne(p[1]), (short)bf16_rne(p[2]),
                     (short)bf16_rne(p[3])};
  const uint16_t *t16 = reinterpret_cast<const uint16_t *>(tile) + kWaveDims * dh;
#pragma unroll
  for (int dt = 0; dt < kWaveDims / 16; ++dt) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) S.O[dt][jj] *= ah[jj];
    v4s vb;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      vb[jj] = (short)t16[((4 * g + jj) * kTileRow) / 2 + 16 * dt + col];
    S.O[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, S.O[dt], 0, 0, 0);
    // keep the V reads of at most four tiles in flight
    if ((dt & 3) == 3) __builtin_amdgcn_sched_barrier(0);
  }
}

__global__ __launch_bounds__(kThreads) void sparse_mla_partial_kernel(MlaArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kBlk * kTileRow];
  // byte offset of each listed row (-1: skipped, or past the chunk, up to
  // the last block loaded ahead)
  __shared__ int64_t row_off[kMlaMaxChunk + (2 * kAhead - 1) * kBlk];
  const int sp = blockIdx.x;
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave & 3; // head group
  const int dh = wave >> 2; // dim half
  const int g = lane >> 4;
  const int col = lane & 15;
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
  const uint16_t *qh = a.q + ((int64_t)r * kMlaHeads + 16 * hg + col) * kMlaDim;
#pragma unroll
  for (int kk = 0; kk < kMlaDim / 32; ++kk)
    S.qb[kk] = *reinterpret_cast<const v8bf *>(qh + 32 * kk + 8 * g);
#pragma unroll
  for (int dt = 0; dt < kWaveDims / 16; ++dt) S.O[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  S.m_run = -__builtin_huge_valf();
  S.l_run = 0.f;
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); // the queries, before any block load is counted
  __syncthreads();                           // the table is complete

  // thread t carries bytes [16 (t & 31), + 16) and [512 + 16 (t & 31), + 16)
  // of row t >> 5 of a block (each load instruction reads two half rows)
  const int gj = tid >> 5;
  const int gs = tid & 31;
  // Loads of block bi; rows past the chunk (and skipped entries) read the
  // cache's first row, inside every valid cache, and are zeroed when stored,
  // so every path keeps the same loads in flight.
  auto load_block = [&](int bi, v4i (&v)[2]) {
    const int64_t off = row_off[bi * kBlk + gj];
    const v4i *src = reinterpret_cast<const v4i *>(a.kv + (off >= 0 ? off : 0) + 16 * gs);
    v[0] = src[0];
    v[1] = src[32];
  };
  auto store_block = [&](int bi, const v4i (&v)[2]) {
    const bool ok = row_off[bi * kBlk + gj] >= 0;
    v4i *dst = reinterpret_cast<v4i *>(tile[bi & 1] + gj * kTileRow + 16 * gs);
    dst[0] = ok ? v[0] : v4i{0, 0, 0, 0};
    dst[32] = ok ? v[1] : v4i{0, 0, 0, 0};
  };
  // One block: store it (its slot was last read two blocks ago, before the
  // previous barrier), publish it, refill its registers three blocks ahead
  // and score it.
  auto step = [&](int bi, v4i (&v)[2]) {
    store_block(bi, v);
    lds_only_barrier();
    load_block(bi + kAhead, v);
    score_block(a, S, tile[bi & 1], dh, row_off + bi * kBlk);
  };

  v4i ra[2], rb[2], rc[2];
  if (nblk > 0) {
    load_block(0, ra);
    load_block(1, rb);
    load_block(2, rc);
    for (int bi = 0; bi < nblk; bi += kAhead) {
      step(bi, ra);
      step(bi + 1, rb);
      step(bi + 2, rc);
    }
  }

  // ---- this chunk's (max, sum, unnormalized O) per head
  const int64_t base = ((int64_t)r * a.nsplit + sp) * kMlaHeads + 16 * hg;
#pragma unroll
  for (int dt = 0; dt < kWaveDims / 16; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      a.ws_o[(base + 4 * g + jj) * kMlaDim + kWaveDims * dh + 16 * dt + col] = S.O[dt][jj];
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
