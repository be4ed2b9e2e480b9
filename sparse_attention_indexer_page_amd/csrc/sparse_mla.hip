// Sparse attention over the indexer's selection on gfx950: every query row
// attends to its own top-k tokens only (flashinfer PR #3269 "Add DeepSeek V4
// sparse MLA TRTLLM-GEN kernels": a decode over dynamic per-row top-k lengths
// with 512-dim QK and V; in MLA the values are the same latent rows as the
// keys). For row r (sequence b = r / next_n), head h and the n_r =
// min(topk_lens[r], k) listed tokens t_i (entries < 0 skipped):
//     s_i = scale * (q[r][h] . c[t_i]),   out[r][h] = sum_i softmax(s)_i c[t_i]
// with c[t] the bf16 latent row of token t through the block table.
//
// Split over tokens (flash decoding): work group (split, r) = 4 waves, wave w
// owning heads 16w..16w+15, scores a contiguous chunk of row r's list in
// blocks of 16 tokens:
//   * the 16 latent rows (16 KB) are gathered through the block table into
//     an LDS tile (rows padded to 1040 bytes, so the four token rows one
//     P.V operand read touches fall in distinct banks);
//   * S^T = K q^T on v_mfma_f32_16x16x32_bf16 (tokens x heads; the wave's 16
//     query heads stay in VGPRs as B operands, 512 dims = 16 k-steps);
//   * online softmax per head; the scores come out of that MFMA in exactly
//     the A-operand layout of the P.V product (lane l: head l & 15, tokens
//     4g..4g+3), so P needs no shuffle, only bf16 rounding;
//   * O += P V on v_mfma_f32_16x16x16_bf16 (heads x 16 dims, K = the 16
//     tokens), 32 tiles for 512 dims, fp32 accumulators in VGPRs.
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
constexpr int kBlk = 16;                  // tokens per block
constexpr int kTileRow = 2 * kMlaDim + 16; // LDS bytes per gathered row

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ inline uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(256) void sparse_mla_partial_kernel(MlaArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kBlk * kTileRow];
  __shared__ int32_t tok_ok[kBlk];
  const int sp = blockIdx.x;
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int col = lane & 15;
  const int b = r / a.next_n;
  int n = uniform_load(a.topk_lens + r);
  n = n < 0 ? 0 : (n > a.k ? a.k : n);
  const int c0 = sp * a.chunk;
  const int c1 = c0 + a.chunk < n ? c0 + a.chunk : n;

  // the wave's 16 query heads as B operands: head 16 wave + col, dims
  // 32 kk + 8 g .. + 8
  v8bf qb[kMlaDim / 32];
  const uint16_t *qh = a.q + ((int64_t)r * kMlaHeads + 16 * wave + col) * kMlaDim;
#pragma unroll
  for (int kk = 0; kk < kMlaDim / 32; ++kk)
    qb[kk] = *reinterpret_cast<const v8bf *>(qh + 32 * kk + 8 * g);

  v4f O[kMlaDim / 16];
#pragma unroll
  for (int dt = 0; dt < kMlaDim / 16; ++dt) O[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_huge_valf(), l_run = 0.f; // head 16 wave + col

  const int gj = tid >> 4; // gathered token of this thread
  const int gs = tid & 15; // its 64-byte segment
  for (int c = c0; c < c1; c += kBlk) {
    // ---- gather 16 latent rows into LDS (zeros for skipped entries)
    const int i = c + gj;
    const int t = i < c1 ? a.indices[(int64_t)r * a.k + i] : -1;
    int64_t pg = -1;
    if (t >= 0) {
      const int64_t lp = t >> a.page_shift;
      if (lp < a.bt_stride) pg = a.block_tables[(int64_t)b * a.bt_stride + lp];
    }
    const bool ok = pg >= 0 && pg < a.num_pages;
    v4i seg[4] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};
    if (ok) {
      const v4i *src = reinterpret_cast<const v4i *>(
          a.kv + pg * a.page_stride + (int64_t)(t & (a.page_size - 1)) * a.row_stride + 64 * gs);
#pragma unroll
      for (int u = 0; u < 4; ++u) seg[u] = src[u];
    }
    v4i *dst = reinterpret_cast<v4i *>(tile + gj * kTileRow + 64 * gs);
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[u] = seg[u];
    if (gs == 0) tok_ok[gj] = ok ? 1 : 0;
    __syncthreads();

    // ---- S^T = K q^T: lane holds head col, tokens 4g..4g+3
    v4f st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kMlaDim / 32; ++kk) {
      const v8bf ka = *reinterpret_cast<const v8bf *>(tile + col * kTileRow + 64 * kk + 16 * g);
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[kk], st, 0, 0, 0);
    }
    // ---- online softmax over the block, per head
    float s[4];
    float bm = -__builtin_huge_valf();
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      s[jj] = tok_ok[4 * g + jj] ? st[jj] * a.scale : -__builtin_huge_valf();
      bm = fmaxf(bm, s[jj]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    const float m_new = fmaxf(m_run, bm);
    const float alpha = m_run == -__builtin_huge_valf() ? 0.f : __expf(m_run - m_new);
    float p[4], ls = 0.f;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      p[jj] = s[jj] == -__builtin_huge_valf() ? 0.f : __expf(s[jj] - m_new);
      ls += p[jj];
    }
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    l_run = l_run * alpha + ls;
    m_run = m_new;
    // O rows are heads 4g + jj: their factors live in lanes 4g + jj
    float ah[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) ah[jj] = __shfl(alpha, 4 * g + jj, 64);
    // P as the A operand: head col, tokens 4g..4g+3, bf16
    const v4s pa = v4s{(short)bf16_rne(p[0]), (short)bf16_rne(p[1]), (short)bf16_rne(p[2]),
                       (short)bf16_rne(p[3])};
    const uint16_t *t16 = reinterpret_cast<const uint16_t *>(tile);
#pragma unroll
    for (int dt = 0; dt < kMlaDim / 16; ++dt) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) O[dt][jj] *= ah[jj];
      v4s vb;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        vb[jj] = (short)t16[((4 * g + jj) * kTileRow) / 2 + 16 * dt + col];
      O[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, O[dt], 0, 0, 0);
    }
    __syncthreads(); // the next gather overwrites the tile
  }

  // ---- this chunk's (max, sum, unnormalized O) per head
  const int64_t base = ((int64_t)r * a.nsplit + sp) * kMlaHeads + 16 * wave;
#pragma unroll
  for (int dt = 0; dt < kMlaDim / 16; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      a.ws_o[(base + 4 * g + jj) * kMlaDim + 16 * dt + col] = O[dt][jj];
  if (g == 0) {
    a.ws_ml[(base + col) * 2] = m_run;
    a.ws_ml[(base + col) * 2 + 1] = l_run;
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
  hipLaunchKernelGGL(sparse_mla_partial_kernel, dim3(a.nsplit, a.R), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sparse_mla_merge_kernel, dim3(kMlaHeads, a.R), dim3(128), 0, s, a);
  return hipGetLastError();
}

} // namespace idx
