// Measurement kernels for the roofline ceilings the indexer kernels are
// compared against on gfx950 (built into libidx_ceilings.so, loaded only by
// `bench.py --ceilings`; not part of the indexer library or its ABI):
//   * paged streaming read: random key pages read once, either gathered in
//     the scoring kernel's MFMA operand order (each 16-byte-per-lane load
//     covers 16 rows x 64 bytes) or as linear 1 KB loads (64 lanes x 16
//     consecutive bytes);
//   * FP8 MFMA issue: 16x16x128 MFMAs alone, the scoring epilogue alone
//     (2*relu(s) as s + |s|, then a multiply-add per score), and both in the
//     scoring kernel's proportion (4 MFMAs per 16 scores per lane).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)n, 0x00020000);
}

// One wave per work group; wave w reads pages[w * ppw .. w * ppw + ppw) of
// ROWS x STRIDE bytes each, one page ahead, and folds the bytes into out.
template <int LINEAR, int ROWS, int STRIDE>
__global__ __launch_bounds__(64) void stream_pages(const uint8_t *pool, const int *pages, int ppw,
                                                   int *out) {
  const int lane = threadIdx.x, g = lane >> 4, col = lane & 15;
  constexpr int PB = ROWS * STRIDE;
  constexpr int NL = LINEAR ? (PB + 1023) / 1024 : (ROWS / 16) * 2;
  const int *pp = pages + (size_t)blockIdx.x * ppw;
  v4i buf[2][NL];
  v4i acc = {0, 0, 0, 0};
  auto issue = [&](int i, v4i(&b)[NL]) {
    const bool live = i < ppw;
    const int pg = live ? pp[i] : 0;
    const __amdgpu_buffer_rsrc_t r = rsrc(pool + (size_t)pg * PB, live ? PB : 0);
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const uint32_t off = LINEAR ? (uint32_t)(1024 * l + 16 * lane)
                                  : (uint32_t)((16 * (l >> 1) + col) * STRIDE + 64 * (l & 1) + 16 * g);
      b[l] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
    }
  };
  issue(0, buf[0]);
  for (int i = 0; i < ppw; i += 2) {
    issue(i + 1, buf[1]);
#pragma unroll
    for (int l = 0; l < NL; ++l) acc ^= buf[0][l];
    issue(i + 2, buf[0]);
#pragma unroll
    for (int l = 0; l < NL; ++l) acc ^= buf[1][l];
  }
  out[blockIdx.x * 64 + lane] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

__device__ inline float relu2(float x) { return x + __builtin_fabsf(x); }

// MODE 0: 8 MFMAs per iteration; 1: the epilogue of 32 scores per lane per
// iteration (32 adds + 32 multiply-adds, on values the compiler must treat as
// new each iteration); 2: both, as the scoring kernel pairs them (the
// epilogue of the previous iteration's MFMA results, two accumulator sets in
// turn).
template <int MODE>
__global__ __launch_bounds__(1024) void mfma_epilogue(const int *in, float *out, int iters) {
  const int lane = threadIdx.x & 63;
  v8i a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = in[(lane * 8 + i) & 1023];
    b[i] = in[(lane * 8 + i + 512) & 1023];
  }
  float w[16];
  for (int i = 0; i < 16; ++i) w[i] = __int_as_float(in[i] & 0x3f7fffff);
  v4f acc[2][8];
  for (int u = 0; u < 2; ++u)
    for (int m = 0; m < 8; ++m) acc[u][m] = v4f{__int_as_float(in[m + u] & 0x3f7fffff), 0.f, 0.f, 0.f};
  float sum = 0.f;
  auto mfmas = [&](v4f(&dst)[8]) { // eight independent accumulations
#pragma unroll
    for (int m = 0; m < 8; ++m)
      dst[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, dst[m], 0, 0, 0, 0, 0, 0);
  };
  auto epilogue = [&](v4f(&src)[8]) {
    if (MODE == 1) {
#pragma unroll
      for (int m = 0; m < 8; ++m) asm volatile("" : "+v"(src[m])); // fresh values each time
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) s = fmaf(w[4 * m + j], relu2(src[4 * t + m][j]), s);
      sum += s;
    }
  };
  for (int it = 0; it < iters; it += 2) {
    if (MODE != 1) mfmas(acc[0]);
    if (MODE != 0) epilogue(acc[1]);
    if (MODE != 1) mfmas(acc[1]);
    if (MODE != 0) epilogue(acc[0]);
    b[1] += it;
  }
  for (int u = 0; u < 2; ++u)
    for (int m = 0; m < 8; ++m) sum += acc[u][m][0] + acc[u][m][1] + acc[u][m][2] + acc[u][m][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

} // namespace

extern "C" {

// Paged read: page_kind 0 = 32 rows x 144 B, 1 = 64 rows x 128 B; linear
// selects the load pattern. Returns a hipError_t value.
int ceil_stream_pages(const void *pool, const int *pages, int pages_per_wave, int waves, int page_kind,
                      int linear, int *out, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t *p = static_cast<const uint8_t *>(pool);
  if (page_kind == 0 && linear)
    hipLaunchKernelGGL((stream_pages<1, 32, 144>), dim3(waves), dim3(64), 0, s, p, pages, pages_per_wave, out);
  else if (page_kind == 0)
    hipLaunchKernelGGL((stream_pages<0, 32, 144>), dim3(waves), dim3(64), 0, s, p, pages, pages_per_wave, out);
  else if (linear)
    hipLaunchKernelGGL((stream_pages<1, 64, 128>), dim3(waves), dim3(64), 0, s, p, pages, pages_per_wave, out);
  else
    hipLaunchKernelGGL((stream_pages<0, 64, 128>), dim3(waves), dim3(64), 0, s, p, pages, pages_per_wave, out);
  return (int)hipGetLastError();
}

// MFMA / epilogue issue loop (mode 0, 1, 2 as above) on `groups` work groups
// of `threads` threads (a multiple of 64, at most 1024). in: 1024 ints whose
// bytes are the FP8 operands (their entropy sets the matrix cores' power
// draw, hence the clock the loop runs at).
int ceil_mfma_epilogue(const int *in, float *out, int iters, int mode, int groups, int threads,
                       void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == 0)
    hipLaunchKernelGGL(mfma_epilogue<0>, dim3(groups), dim3(threads), 0, s, in, out, iters);
  else if (mode == 1)
    hipLaunchKernelGGL(mfma_epilogue<1>, dim3(groups), dim3(threads), 0, s, in, out, iters);
  else
    hipLaunchKernelGGL(mfma_epilogue<2>, dim3(groups), dim3(threads), 0, s, in, out, iters);
  return (int)hipGetLastError();
}

} // extern "C"
