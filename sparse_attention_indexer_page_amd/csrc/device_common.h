// Device helpers shared by the gfx950 scoring kernels (decode and prefill).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idx {
namespace dev {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kFmtFp8 = 0; // f8f6f4 format code: E4M3
constexpr int kFmtFp4 = 4; // f8f6f4 format code: E2M1

// Raw buffer resource word 3 for gfx9: no swizzle, no format conversion.
constexpr int kRsrcWord3 = 0x00020000;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

__device__ inline v4i load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ inline uint32_t load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// 2 * max(x, 0), exactly: x + |x| is 2x for x > 0 and +0 otherwise, and
// doubling is exact. One add with an abs source modifier, a full-rate VALU
// op on gfx950, where an integer or float max issues at about half that rate
// (measured: 1.1 vs 1.8 ns per wave64 op per SIMD). The scoring epilogues
// sum w * relu2(s) and halve the head sum once per token, which gives the
// same bits as summing w * max(s, 0): every partial sum is exactly twice as
// large (barring overflow and subnormal results).
__device__ inline float relu2(float x) { return x + __builtin_fabsf(x); }

// s_waitcnt immediate that waits until at most n vector-memory operations
// of the wave are outstanding (gfx9 layout: vmcnt in bits [3:0] and [15:14];
// expcnt (7) and lgkmcnt (15) left unwaited).
__device__ inline constexpr int waitcnt_vm(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// s_waitcnt immediate that waits for every outstanding LDS and scalar-memory
// operation of the wave (lgkmcnt 0; vmcnt and expcnt left unwaited).
__device__ inline constexpr int waitcnt_lgkm0() { return 15 | (3 << 14) | (7 << 4); }

// Wave-uniform read of launch metadata (lengths, block-table entries, the
// work schedule) through the scalar cache: a constant-address-space load at a
// uniform address becomes s_load, counted by lgkmcnt, so waiting for it never
// waits for the wave's outstanding vector-memory loads or stores. The data
// must not change while the kernel runs.
template <typename T> __device__ inline T uniform_load(const T *p) {
  return *(const __attribute__((address_space(4))) T *)p;
}

// Storage-format encoders shared by the K-cache writer and the query
// quantizer (see those kernels for the per-row / per-block scale rules).
// Nearest E4M3FN code to y (|y| <= 448 up to rounding), ties to the even code.
__device__ inline uint32_t fp8_e4m3_rne(float y) {
  const uint32_t b = __float_as_uint(y);
  const uint32_t sign = (b >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t code;
  if (a < 0.015625f) {
    // subnormal range: multiples of 2^-9; rintf rounds half to even
    code = (uint32_t)rintf(a * 512.0f); // 8 means the smallest normal, 0x08
  } else {
    // normal: keep 3 mantissa bits of the fp32 pattern, round half to even
    const uint32_t ab = __float_as_uint(a);
    const uint32_t lsb = (ab >> 20) & 1u;
    const uint32_t r = ab + 0x7FFFFu + lsb;        // may carry into the exponent
    const uint32_t exp = (r >> 23) - 127 + 7;      // E4M3 biased exponent
    code = (exp << 3) | ((r >> 20) & 7u);
    if (code > 0x7Eu) code = 0x7Eu; // saturate at 448
  }
  return code | sign;
}

// Nearest E2M1 magnitude code (0..7) to a >= 0, ties to the even code,
// saturating at 6.
__device__ inline uint32_t e2m1_rne(float a) {
  return (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) +
         (a > 5.0f);
}

// OCP MX shared exponent of a block with magnitude maximum m:
// floor(log2 m) - 2 (2 = the largest E2M1 exponent), clamped to [-127, 127];
// 0 for an all-zero block. The E8M0 byte is the result + 127.
__device__ inline int mx_block_exponent(float m) {
  if (!(m > 0.f)) return 0;
  int ex;
  (void)frexpf(m, &ex); // m = f * 2^ex, f in [0.5, 1)
  const int e = ex - 1 - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__device__ inline v8i cat(v4i a, v4i b) { return v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}; }

// Sum over lane groups g = lane >> 4 of per-lane partials p[t] (one per tile),
// scattered so that group g ends with tile g's column totals (TPB = 4), or
// groups 2t and 2t+1 both with tile t's (TPB = 2). Uses the gfx950 row swaps
// (v_permlane32_swap: upper 32 lanes of x <-> lower 32 of y; v_permlane16_swap:
// odd 16-lane rows of x <-> even rows of y), so no LDS traffic.
template <int TPB> __device__ inline float reduce_scatter(const float (&p)[TPB]);

template <> __device__ inline float reduce_scatter<4>(const float (&p)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[2]),
                                                  false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[1]), __float_as_uint(p[3]),
                                                  false, false);
  // lanes 0-31 now sum tiles 0 / 1 over both halves, lanes 32-63 tiles 2 / 3
  const float sa = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float sb = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(sa), __float_as_uint(sb), false,
                                                  false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

template <> __device__ inline float reduce_scatter<2>(const float (&p)[2]) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[1]),
                                                  false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false,
                                                  false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

} // namespace dev
} // namespace idx
