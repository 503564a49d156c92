// kvq_device.h -- device-side helpers shared by the library's HIP kernels.
//
// Every helper that feeds a decision (a code, a selection, a verdict, a
// level) uses fp32 with round-to-nearest-even, explicit fmaf and no
// contraction (the library is built with -ffp-contract=off and fp32
// denormals kept), so results are reproducible bit for bit.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace kvq {

constexpr int BLOCK = 64;   // tokens per block
constexpr int VGROUP = 32;  // channels per value group

__device__ __forceinline__ float h2f(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}
__device__ __forceinline__ uint16_t f2h(float f) {  // round to nearest even
  return __half_as_ushort(__float2half_rn(f));
}
// Binary16 scale rounded up: the nearest binary16, stepped one ulp up when
// it fell below q (q >= 0).  The stored scale never undershoots the range.
__device__ __forceinline__ uint16_t ru16(float q) {
  uint16_t h = f2h(q);
  if (h2f(h) < q) h = (uint16_t)(h + 1);
  return h;
}

// Base-2 exponential used by every decision: round x to the nearest integer
// n, f = x - n (exact, |f| <= 1/2), 2^f by its degree-7 Taylor polynomial
// (coefficients (ln 2)^k / k! rounded to binary32) in Horner form with fmaf,
// scaled by 2^n.  Zero for x < -125 (results are always normal otherwise).
__device__ __forceinline__ float exp2k(float x) {
  if (!(x >= -125.0f)) return 0.0f;
  float n = rintf(x);
  float f = x - n;
  float p = 0x1.ffcbfcp-17f;           // (ln2)^7/7!
  p = fmaf(p, f, 0x1.430912p-13f);     // (ln2)^6/6!
  p = fmaf(p, f, 0x1.5d87fep-10f);     // (ln2)^5/5!
  p = fmaf(p, f, 0x1.3b2ab6p-7f);      // (ln2)^4/4!
  p = fmaf(p, f, 0x1.c6b08ep-5f);      // (ln2)^3/3!
  p = fmaf(p, f, 0x1.ebfbe0p-3f);      // (ln2)^2/2!
  p = fmaf(p, f, 0x1.62e430p-1f);      // ln2
  p = fmaf(p, f, 1.0f);
  return ldexpf(p, (int)n);
}

// floor(log2 |x|) for finite nonzero x (subnormals included).
__device__ __forceinline__ int ilogb_f(float x) {
  int e;
  (void)frexpf(x, &e);
  return e - 1;
}

// Order-preserving map of floats to unsigned ints (for atomic min/max).
__device__ __forceinline__ uint32_t f_ord(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f_unord(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

__device__ __forceinline__ float nextup_pos(float x) {
  return __uint_as_float(__float_as_uint(x) + 1u);
}

// int64 -> fp32, one rounding (|v| < 2^53 is exact in fp64 first).
__device__ __forceinline__ float i64_to_f32(long long v) {
  return (float)(double)v;
}

// Butterfly reductions over lanes that differ in the low bits given by MASKS
// (xor partners).  For sums this realises fold-in-half: the pair (j, j^w)
// adds the same two values in either lane (fp32 addition is commutative).
template <int W>
__device__ __forceinline__ float bfly_sum(float v) {
#pragma unroll
  for (int w = W / 2; w >= 1; w >>= 1) v = v + __shfl_xor(v, w, 64);
  return v;
}
template <int W>
__device__ __forceinline__ float bfly_max(float v) {
#pragma unroll
  for (int w = W / 2; w >= 1; w >>= 1) v = fmaxf(v, __shfl_xor(v, w, 64));
  return v;
}
template <int W>
__device__ __forceinline__ uint32_t bfly_sum_u32(uint32_t v) {
#pragma unroll
  for (int w = W / 2; w >= 1; w >>= 1) v += (uint32_t)__shfl_xor((int)v, w, 64);
  return v;
}

// Wave-level LDS hand-off between lanes of one wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

}  // namespace kvq
