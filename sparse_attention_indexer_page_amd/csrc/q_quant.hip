// Query-side quantization with the weight fold on gfx950: the step before the
// scores (ROCm/ATOM PR #1709: the indexer's forward_pre returns the quantized
// q and the per-head weights that score_topk_from consumes).
//
// One work group of 256 threads per query row of 64 heads x 128 values; each
// thread quantizes 8 consecutive values in each of four passes (2048 values
// per pass, so loads and stores stay contiguous across the group).
//   * FP8 E4M3FN: one scale per row, s = amax/448 over all 8192 values (1 for
//     an all-zero row), codes = x/s rounded to the nearest E4M3 value (ties
//     to even, sign kept) -- the K-cache writer's rule on a longer row. The
//     weights become w*s*c (single-precision products, in that order) when no
//     q scale output is given, folding s away; with a q scale output they
//     become w*c and s is written there.
//   * MXFP4: per 32 values (four threads) the OCP MX exponent and E2M1 codes as
//     the K-cache writer, codes to [64][64] bytes (even value in the low
//     nibble), E8M0 bytes to [64][4]; the weights become w*c.
// The codes are stored with the non-temporal hint: nothing reads them back
// before the scoring launch, and the 16384-row batch then takes 95 us
// instead of 100 (measured).
#include "device_common.h"
#include "internal.h"

namespace idx {
namespace {

using namespace dev;

constexpr int kThreads = 256;
constexpr int kRowValues = kHeads * kHeadDim; // 8192
constexpr int kPerThread = 8;
constexpr int kPasses = kRowValues / (kThreads * kPerThread); // 4

typedef uint32_t v2u __attribute__((ext_vector_type(2)));

__device__ inline void load8(const QQuantArgs &a, int64_t i, float (&x)[8]) {
  if (a.x_bf16) {
    const v4i v = *reinterpret_cast<const v4i *>(reinterpret_cast<const uint16_t *>(a.x) + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float((uint32_t)v[j] << 16);
      x[2 * j + 1] = __uint_as_float((uint32_t)v[j] & 0xFFFF0000u);
    }
  } else {
    const v4f v0 = *reinterpret_cast<const v4f *>(reinterpret_cast<const float *>(a.x) + i);
    const v4f v1 = *reinterpret_cast<const v4f *>(reinterpret_cast<const float *>(a.x) + i + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = v0[j];
      x[4 + j] = v1[j];
    }
  }
}

__global__ __launch_bounds__(kThreads) void q_quant_kernel(QQuantArgs a) {
  __shared__ float red[kThreads / 64];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  float x[kPasses][8];
  const int64_t base = (int64_t)r * a.x_row_stride;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) load8(a, base + p * (kThreads * kPerThread) + kPerThread * tid, x[p]);
  const float *w = a.w + (int64_t)r * kHeads;
  float *wo = a.w_out + (int64_t)r * kHeads;
  if (a.dtype == IDX_FP8_E4M3) {
    float m = 0.f;
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[p][j]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = m > 0.f ? m / 448.0f : 1.0f;
    uint8_t *q = a.q + (int64_t)r * kRowValues;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lo |= fp8_e4m3_rne(x[p][j] / s) << (8 * j);
        hi |= fp8_e4m3_rne(x[p][4 + j] / s) << (8 * j);
      }
      __builtin_nontemporal_store(
          v2u{lo, hi}, reinterpret_cast<v2u *>(q + p * (kThreads * kPerThread) + kPerThread * tid));
    }
    if (tid < kHeads) {
      if (a.q_scale) {
        wo[tid] = w[tid] * a.c;
        if (tid == 0) reinterpret_cast<float *>(a.q_scale)[r] = s;
      } else {
        wo[tid] = (w[tid] * s) * a.c;
      }
    }
  } else {
    uint8_t *q = a.q + (int64_t)r * (kRowValues / 2);
    uint8_t *qs = a.q_scale + (int64_t)r * (kRowValues / 32);
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      float m = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[p][j]));
      m = fmaxf(m, __shfl_xor(m, 1, 64)); // the block's four threads
      m = fmaxf(m, __shfl_xor(m, 2, 64));
      const int e = mx_block_exponent(m);
      uint32_t packed = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float y = ldexpf(x[p][j], -e);
        uint32_t c = e2m1_rne(fabsf(y));
        if (y < 0.f && c) c |= 8u;
        packed |= c << (4 * j);
      }
      const int v0 = p * (kThreads * kPerThread) + kPerThread * tid; // first value
      __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t *>(q + v0 / 2));
      if ((tid & 3) == 0) qs[v0 / 32] = (uint8_t)(e + 127);
    }
    if (tid < kHeads) wo[tid] = w[tid] * a.c;
  }
}

} // namespace

hipError_t launch_q_quant(const QQuantArgs &a, hipStream_t s) {
  if (a.R <= 0) return hipSuccess;
  hipLaunchKernelGGL(q_quant_kernel, dim3(a.R), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

} // namespace idx
