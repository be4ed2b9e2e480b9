// Indexer K-cache writer on gfx950: new key rows are quantized to the cache's
// storage format and scattered into their pages (ROCm/ATOM PR #1709 names the
// "FP4 mqa-logits / scatter kernels" in the commit adding the FP4 indexer
// flag; the scores read exactly what this writes).
//
// One wave per row of 128 values, two per lane (elements 2l and 2l+1):
//   * FP8 E4M3FN: one fp32 scale per row, amax / 448 (1 for an all-zero row);
//     each code is x / scale rounded to the nearest E4M3 value, ties to the
//     even code, sign kept. Lane l stores bytes 2l, 2l+1 (a coalesced 128-byte
//     row) and lane 0 the scale.
//   * MXFP4 (OCP MX): per 32-element block (16 lanes) the shared exponent
//     e = floor(log2 amax) - 2 (the largest E2M1 exponent), clamped to
//     [-127, 127], 0 for an all-zero block; codes are |x| * 2^-e rounded to the
//     nearest E2M1 magnitude, ties to the even code, saturating at 6, sign only
//     on a nonzero code. Lane l stores byte l (element 2l in the low nibble);
//     lane 0 stores the four E8M0 bytes.
// slot_mapping[t] = page * P + slot places row t; a negative slot or a page
// outside the pool skips the row (nothing is written).
#include "device_common.h"
#include "internal.h"

namespace idx {
namespace {

using namespace dev;

constexpr int kRowsPerGroup = 4; // waves per work group
constexpr int kRowsPerWave = 4;

// Elements i and i+1 (i even) of the input, as fp32, with one load.
__device__ inline void load_pair(const KvWriteArgs &a, int64_t i, float &x0, float &x1) {
  if (a.k_bf16) {
    const uint32_t h = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(a.k) + i);
    x0 = __uint_as_float(h << 16);
    x1 = __uint_as_float(h & 0xFFFF0000u);
  } else {
    const float2 v = *reinterpret_cast<const float2 *>(reinterpret_cast<const float *>(a.k) + i);
    x0 = v.x;
    x1 = v.y;
  }
}

// Quantizes one row (x0, x1 = this lane's two values) into its slot.
__device__ inline void write_row(const KvWriteArgs &a, int64_t slot, float x0, float x1) {
  const int lane = threadIdx.x & 63;
  if (slot < 0) return;
  const int64_t pg = slot >> a.page_shift;
  const int64_t sl = slot & ((1 << a.page_shift) - 1);
  if (pg >= a.num_pages) return;
  uint8_t *row = a.data + pg * a.page_stride + sl * a.row_stride;
  uint8_t *srow = a.scale + pg * a.scale_page_stride + sl * a.scale_row_stride;
  float m = fmaxf(fabsf(x0), fabsf(x1));
  if (a.dtype == IDX_FP8_E4M3) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    const float s = m > 0.f ? m / 448.0f : 1.0f;
    const uint32_t c0 = fp8_e4m3_rne(x0 / s), c1 = fp8_e4m3_rne(x1 / s);
    reinterpret_cast<uint16_t *>(row)[lane] = (uint16_t)(c0 | (c1 << 8));
    if (lane == 0) *reinterpret_cast<float *>(srow) = s;
  } else {
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64)); // 16-lane block
    const int e = mx_block_exponent(m);
    const float y0 = ldexpf(x0, -e), y1 = ldexpf(x1, -e);
    uint32_t c0 = e2m1_rne(fabsf(y0)), c1 = e2m1_rne(fabsf(y1));
    if (y0 < 0.f && c0) c0 |= 8u;
    if (y1 < 0.f && c1) c1 |= 8u;
    row[lane] = (uint8_t)(c0 | (c1 << 4));
    const uint32_t sb = (uint32_t)(e + 127);
    const uint32_t s0 = __builtin_amdgcn_readlane(sb, 0), s1 = __builtin_amdgcn_readlane(sb, 16);
    const uint32_t s2 = __builtin_amdgcn_readlane(sb, 32), s3 = __builtin_amdgcn_readlane(sb, 48);
    if (lane == 0) {
      srow[0] = (uint8_t)s0;
      srow[1] = (uint8_t)s1;
      srow[2] = (uint8_t)s2;
      srow[3] = (uint8_t)s3;
    }
  }
}

// Each wave takes kRowsPerWave consecutive rows and loads all of them before
// quantizing any, so the load latency is paid once per group of rows.
__global__ __launch_bounds__(64 * kRowsPerGroup) void kv_write_kernel(KvWriteArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int t0 = (blockIdx.x * kRowsPerGroup + wave) * kRowsPerWave;
  if (t0 >= a.N) return;
  float x0[kRowsPerWave], x1[kRowsPerWave];
  int64_t slot[kRowsPerWave];
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) {
    const int t = t0 + j < a.N ? t0 + j : a.N - 1; // past the end: reload the last row
    load_pair(a, (int64_t)t * a.k_row_stride + 2 * lane, x0[j], x1[j]);
    slot[j] = t0 + j < a.N ? uniform_load(a.slot_mapping + t) : -1;
  }
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) write_row(a, slot[j], x0[j], x1[j]);
}

} // namespace

hipError_t launch_kv_write(const KvWriteArgs &a, hipStream_t s) {
  if (a.N <= 0) return hipSuccess;
  const int per_group = kRowsPerGroup * kRowsPerWave;
  const int groups = (a.N + per_group - 1) / per_group;
  hipLaunchKernelGGL(kv_write_kernel, dim3(groups), dim3(64 * kRowsPerGroup), 0, s, a);
  return hipGetLastError();
}

} // namespace idx
