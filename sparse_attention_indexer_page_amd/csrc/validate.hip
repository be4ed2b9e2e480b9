// Device-side check of the decode contracts the host cannot check without a
// sync (the explicit-errors discipline of flashinfer PR #3269's review, and
// ATOM PR #1709's ragged-window commit, where stale lengths and page ids
// turned into a memory fault): every sequence's length within the logits
// width and the block table, and every block-table entry of a page that
// holds a visible token naming a page of the pool. The result lands in a
// caller-owned int32[4] on the stream; nothing synchronizes.
//   result[0] sequences whose length is negative, above W or above the
//             table's bt_cols * page_size tokens
//   result[1] block-table entries of visible pages outside [0, num_pages)
//   result[2] first such sequence (or -1)
//   result[3] sequence of the first such entry (or -1)
#include "device_common.h"
#include "internal.h"

namespace idx {
namespace {

constexpr int kThreads = 256;

// Clears the result (a kernel rather than a memset, so graph replays
// re-run it).
__global__ __launch_bounds__(64) void validate_init_kernel(int32_t *result) {
  if (threadIdx.x < 2) result[threadIdx.x] = 0;
  else if (threadIdx.x < 4) result[threadIdx.x] = 0x7FFFFFFF;
}

// One work group per sequence.
__global__ __launch_bounds__(kThreads) void validate_decode_kernel(ValidateArgs a) {
  const int b = blockIdx.x;
  const int32_t len = a.lens[b];
  const int64_t cap = (int64_t)a.bt_cols * a.page_size;
  const bool bad_len = len < 0 || (a.W > 0 && len > a.W) || len > cap;
  if (bad_len && threadIdx.x == 0) {
    atomicAdd(&a.result[0], 1);
    atomicMin(&a.result[2], b);
  }
  int64_t pages = len > 0 ? ((int64_t)len + a.page_size - 1) / a.page_size : 0;
  pages = pages < a.bt_cols ? pages : a.bt_cols;
  int32_t bad = 0;
  for (int64_t p = threadIdx.x; p < pages; p += kThreads) {
    const int64_t id = a.block_tables[(int64_t)b * a.bt_stride + p];
    bad += (id < 0 || id >= a.num_pages) ? 1 : 0;
  }
  if (bad != 0) {
    atomicAdd(&a.result[1], bad);
    atomicMin(&a.result[3], b);
  }
}

// -1 for "none" once every sequence is checked.
__global__ __launch_bounds__(64) void validate_finish_kernel(int32_t *result) {
  if (threadIdx.x >= 2 && threadIdx.x < 4 && result[threadIdx.x] == 0x7FFFFFFF)
    result[threadIdx.x] = -1;
}

} // namespace

hipError_t launch_validate_decode(const ValidateArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(validate_init_kernel, dim3(1), dim3(64), 0, s, a.result);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.B > 0) {
    hipLaunchKernelGGL(validate_decode_kernel, dim3(a.B), dim3(kThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(validate_finish_kernel, dim3(1), dim3(64), 0, s, a.result);
  return hipGetLastError();
}

} // namespace idx
