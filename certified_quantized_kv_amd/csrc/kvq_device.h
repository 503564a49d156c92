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
// Evaluated without a branch: the argument is clamped before the polynomial
// and the result selected afterwards (identical values for every x).
__device__ __forceinline__ float exp2k(float x) {
  const float xc = fmaxf(x, -126.0f);  // NaN -> -126, result discarded below
  const float n = rintf(xc);
  const float f = xc - n;
  float p = 0x1.ffcbfcp-17f;           // (ln2)^7/7!
  p = fmaf(p, f, 0x1.430912p-13f);     // (ln2)^6/6!
  p = fmaf(p, f, 0x1.5d87fep-10f);     // (ln2)^5/5!
  p = fmaf(p, f, 0x1.3b2ab6p-7f);      // (ln2)^4/4!
  p = fmaf(p, f, 0x1.c6b08ep-5f);      // (ln2)^3/3!
  p = fmaf(p, f, 0x1.ebfbe0p-3f);      // (ln2)^2/2!
  p = fmaf(p, f, 0x1.62e430p-1f);      // ln2
  p = fmaf(p, f, 1.0f);
  const float r = ldexpf(p, (int)n);
  return (x >= -125.0f) ? r : 0.0f;
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

__device__ __forceinline__ float nextup_pos(float x) {
  return __uint_as_float(__float_as_uint(x) + 1u);
}

// Smallest float >= x for x >= 0 (a bound rounded up to binary32).
__device__ __forceinline__ float f32_up(double x) {
  float f = (float)x;
  if ((double)f < x) f = __uint_as_float(__float_as_uint(f) + 1u);
  return f;
}

// int64 -> fp32, one rounding (|v| < 2^53 is exact in fp64 first).
__device__ __forceinline__ float i64_to_f32(long long v) {
  return (float)(double)v;
}

// Value of lane j ^ X for every lane j (X a power of two below 64).  Within a
// row of 16 lanes the exchange is done by DPP moves (quad permutes, the
// half-row mirror, the row rotate by 8), across rows by the CDNA4 lane swaps
// v_permlane16_swap (rows 0 <-> 1, 2 <-> 3) and v_permlane32_swap (lanes
// 0..31 <-> 32..63): all on the vector ALU, none through LDS.
template <int X>
__device__ __forceinline__ int xor_lane(int v) {
  static_assert(X == 1 || X == 2 || X == 4 || X == 8 || X == 16 || X == 32, "lane xor");
  if constexpr (X == 1) {
    return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xf, 0xf, false);    // quad_perm [1,0,3,2]
  } else if constexpr (X == 2) {
    return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xf, 0xf, false);    // quad_perm [2,3,0,1]
  } else if constexpr (X == 4) {
    // half-row mirror (j ^ 7), then quad_perm [3,2,1,0] (j ^ 3)
    const int t = __builtin_amdgcn_mov_dpp(v, 0x141, 0xf, 0xf, false);
    return __builtin_amdgcn_mov_dpp(t, 0x1B, 0xf, 0xf, false);
  } else if constexpr (X == 8) {
    return __builtin_amdgcn_mov_dpp(v, 0x128, 0xf, 0xf, false);   // row_ror:8
  } else if constexpr (X == 16) {
    // the swap leaves the partner's value in the first result on odd rows
    // and in the second on even rows
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (__lane_id() & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (__lane_id() & 32) ? r[0] : r[1];
  }
}
template <int X>
__device__ __forceinline__ unsigned long long xor_lane_u64(unsigned long long v) {
  const int lo = xor_lane<X>((int)(uint32_t)v);
  const int hi = xor_lane<X>((int)(uint32_t)(v >> 32));
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8
// inside each row of 16 lanes (DPP row_shr, zero shifted in), then the last
// lane of row 0 is added to row 1 and of row 2 to row 3 (row_bcast:15), and
// the last lane of row 1 to rows 2 and 3 (row_bcast:31).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
  const uint32_t lo = dpp_u32<CTRL, ROWS>((uint32_t)v), hi = dpp_u32<CTRL, ROWS>((uint32_t)(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  x += dpp_u32<0x111, 0xf>(x);
  x += dpp_u32<0x112, 0xf>(x);
  x += dpp_u32<0x114, 0xf>(x);
  x += dpp_u32<0x118, 0xf>(x);
  x += dpp_u32<0x142, 0xa>(x);
  x += dpp_u32<0x143, 0xc>(x);
  return x;
}
__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long x) {
  x += dpp_u64<0x111, 0xf>(x);
  x += dpp_u64<0x112, 0xf>(x);
  x += dpp_u64<0x114, 0xf>(x);
  x += dpp_u64<0x118, 0xf>(x);
  x += dpp_u64<0x142, 0xa>(x);
  x += dpp_u64<0x143, 0xc>(x);
  return x;
}

// Butterfly reductions of integers over the 64 lanes (result in every lane).
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
  v += xor_lane_u64<32>(v);
  v += xor_lane_u64<16>(v);
  v += xor_lane_u64<8>(v);
  v += xor_lane_u64<4>(v);
  v += xor_lane_u64<2>(v);
  v += xor_lane_u64<1>(v);
  return v;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  v = max(v, xor_lane_u64<32>(v));
  v = max(v, xor_lane_u64<16>(v));
  v = max(v, xor_lane_u64<8>(v));
  v = max(v, xor_lane_u64<4>(v));
  v = max(v, xor_lane_u64<2>(v));
  v = max(v, xor_lane_u64<1>(v));
  return v;
}
__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) {
  v = min(v, xor_lane_u64<32>(v));
  v = min(v, xor_lane_u64<16>(v));
  v = min(v, xor_lane_u64<8>(v));
  v = min(v, xor_lane_u64<4>(v));
  v = min(v, xor_lane_u64<2>(v));
  v = min(v, xor_lane_u64<1>(v));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)xor_lane<32>((int)v));
  v = max(v, (uint32_t)xor_lane<16>((int)v));
  v = max(v, (uint32_t)xor_lane<8>((int)v));
  v = max(v, (uint32_t)xor_lane<4>((int)v));
  v = max(v, (uint32_t)xor_lane<2>((int)v));
  v = max(v, (uint32_t)xor_lane<1>((int)v));
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)xor_lane<32>((int)v));
  v = min(v, (uint32_t)xor_lane<16>((int)v));
  v = min(v, (uint32_t)xor_lane<8>((int)v));
  v = min(v, (uint32_t)xor_lane<4>((int)v));
  v = min(v, (uint32_t)xor_lane<2>((int)v));
  v = min(v, (uint32_t)xor_lane<1>((int)v));
  return v;
}
__device__ __forceinline__ int wave_min_i32(int v) {
  v = min(v, xor_lane<32>(v));
  v = min(v, xor_lane<16>(v));
  v = min(v, xor_lane<8>(v));
  v = min(v, xor_lane<4>(v));
  v = min(v, xor_lane<2>(v));
  v = min(v, xor_lane<1>(v));
  return v;
}
template <int X>
__device__ __forceinline__ float xor_lane_f(float v) {
  return __int_as_float(xor_lane<X>(__float_as_int(v)));
}

// Butterfly reductions over groups of W lanes (xor partners W/2, ..., 1).
// For sums this realises fold-in-half: the pair (j, j^w) adds the same two
// values in either lane (fp32 addition is commutative).
template <int W>
__device__ __forceinline__ float bfly_sum(float v) {
  if constexpr (W > 1) {
    v = v + xor_lane_f<W / 2>(v);
    return bfly_sum<W / 2>(v);
  }
  return v;
}
template <int W>
__device__ __forceinline__ float bfly_max(float v) {
  if constexpr (W > 1) {
    v = fmaxf(v, xor_lane_f<W / 2>(v));
    return bfly_max<W / 2>(v);
  }
  return v;
}
template <int W>
__device__ __forceinline__ uint32_t bfly_sum_u32(uint32_t v) {
  if constexpr (W > 1) {
    v += (uint32_t)xor_lane<W / 2>((int)v);
    return bfly_sum_u32<W / 2>(v);
  }
  return v;
}

// Wave-level LDS hand-off between lanes of one wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

}  // namespace kvq
