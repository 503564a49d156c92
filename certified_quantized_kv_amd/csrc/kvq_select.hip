// kvq_select.hip -- top-K* coverage selection and promotion planning
// ("Runtime-Certified Bounded-Error Quantized Attention", Méthodologie §3:
// the top-K* blocks covering tau_cov of the estimated mass get FP16 keys).
//
// Per query head: fixed-point INT8 block weights
//   What_b = floor(fl32(fl32(Lhat_b) exp2k(fl32(mhat_b - max_b mhat_b))))  (< 2^31)
// are sorted by (What descending, block index ascending) as 64-bit keys
// What << 32 | ~b (bucket sort in LDS), prefix-summed in 64-bit integers, and
//   K* = min k >= 1 with 10^6 sum_{i<k} What_pi(i) >= tau_ppm sum_b What_b.
// Integer sums make the result independent of reduction order.
// Promotion is per KV head: U_g = union of the group's top-K* sets.  Each
// head's workgroup marks its blocks in U_g and in the group's new-block
// flags; the host reads U back and copies its runs of consecutive blocks.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_blockops.h"

namespace kvq {

constexpr int SEL_NT = 1024;

// EB = blocks per thread (the launch picks the least that covers the
// longest sequence of the call).
template <int EB>
__global__ __launch_bounds__(SEL_NT) void k_select(Shape s, Step w, SeqTab tab, int tau_ppm) {
  extern __shared__ unsigned long long keys[];
  __shared__ float red[SEL_NT / 64];
  __shared__ unsigned long long sbuf[SEL_NT / 64];
  const int i = blockIdx.y, hq = blockIdx.x;
  const int T = tab.T[i], NB = (T + BLOCK - 1) / BLOCK;
  const int n2 = max(64, pow2_at_least(NB));
  const size_t base = ((size_t)i * s.Hq + hq) * s.NBmax;

  // the thread's blocks b = t + r SEL_NT, loaded once
  float mh[EB];
  uint32_t lh[EB];
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < EB; ++r) {
    const int b = threadIdx.x + r * SEL_NT;
    if (b < NB) {
      mh[r] = w.mhat[base + b];
      lh[r] = w.Lhat[base + b];
      m = fmaxf(m, mh[r]);
    }
  }
  m = bfly_max<64>(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  const float M = wave_partials_max_f32(red, SEL_NT / 64);

  // the keys stay in registers for the sort (and go to LDS for its
  // comparison-network fallback)
  unsigned long long kv[EB];
#pragma unroll
  for (int r = 0; r < EB; ++r) {
    const int b = threadIdx.x + r * SEL_NT;
    kv[r] = 0ull;
    if (b < NB) {
      const uint32_t W = (uint32_t)floorf((float)lh[r] * exp2k(mh[r] - M));
      w.What[base + b] = W;
      kv[r] = ((unsigned long long)W << 32) | (unsigned long long)(0xffffffffu - (uint32_t)b);
    }
    if (b < n2) keys[b] = kv[r];
  }
  sort_desc_u64_regs<SEL_NT, EB>(kv, keys, NB, n2);

  // pi, then prefix sums of the sorted weights: thread t owns positions
  // [t*per, (t+1)*per)
  constexpr int PMAX = (MAX_NB + SEL_NT - 1) / SEL_NT;
  const int per = (NB + SEL_NT - 1) / SEL_NT;
  const int p0 = threadIdx.x * per;
  unsigned long long own = 0ull;
  uint32_t wk[PMAX];                            // the weights at the thread's positions
#pragma unroll
  for (int k = 0; k < PMAX; ++k) {
    const int p = p0 + k;
    wk[k] = 0u;
    if (k < per && p < NB) {
      const unsigned long long key = keys[p];
      w.pi[base + p] = 0xffffffffu - (uint32_t)(key & 0xffffffffull);
      wk[k] = (uint32_t)(key >> 32);
      own += wk[k];
    }
  }
  unsigned long long total;
  // (sbuf is not written again: no barrier after the scan)
  const unsigned long long incl = block_incl_scan_u64<SEL_NT, false>(own, sbuf, &total);
  // 10^6 pre >= tau_ppm total  <=>  pre >= ceil(tau_ppm total / 10^6)
  // (integers below 2^63), so each candidate costs one 64-bit compare
  const unsigned long long need = ((unsigned long long)tau_ppm * total + 999999ull) / 1000000ull;
  __shared__ int kst;
  unsigned long long pre = incl - own;
#pragma unroll
  for (int k = 0; k < PMAX; ++k) {
    const int p = p0 + k;                       // K* candidate p + 1
    if (k >= per || p >= NB) break;
    const bool ok_prev = (p == 0) ? false : (pre >= need);
    pre += wk[k];
    const bool ok = pre >= need;
    if (ok && !ok_prev) {
      w.k0[(size_t)i * s.Hq + hq] = p + 1;
      w.ssize[(size_t)i * s.Hq + hq] = p + 1;
      kst = p + 1;
    }
  }
  __syncthreads();

  // the head's selection joins U_g and the group's new blocks (U is empty at
  // this point of the step, so every selected block is new)
  const int g = hq / s.G;
  const size_t ig = (size_t)i * s.Hkv + g;
  uint8_t *Kn = w.Knew + ig * s.NBmax;
  uint8_t *Ug = w.U + ig * s.NBmax;
  for (int p = threadIdx.x; p < kst; p += SEL_NT) {
    const uint32_t b = 0xffffffffu - (uint32_t)(keys[p] & 0xffffffffull);
    Kn[b] = 1;      // benign races across the group's heads: every writer stores 1
    Ug[b] = 1;
  }
}

hipError_t launch_select(const Shape &s, const Step &w, const SeqTab &tab, int tau_ppm, int maxNB,
                         hipStream_t st) {
  const int n2 = max(64, pow2_at_least(maxNB));
  const dim3 grid(s.Hq, tab.n), block(SEL_NT);
  const uint32_t lds = (uint32_t)sort_lds_bytes(n2);
  switch ((maxNB + SEL_NT - 1) / SEL_NT) {
    case 1: return launch_k(k_select<1>, grid, block, lds, st, s, w, tab, tau_ppm);
    case 2: return launch_k(k_select<2>, grid, block, lds, st, s, w, tab, tau_ppm);
    case 3: return launch_k(k_select<3>, grid, block, lds, st, s, w, tab, tau_ppm);
    default: return launch_k(k_select<4>, grid, block, lds, st, s, w, tab, tau_ppm);
  }
}

// The workgroup sort of the selection and controller kernels on n distinct
// nonzero keys (cap = max(64, next power of two >= n), unused slots zero);
// *path = 0 when the bucket sort placed the keys, 1 when the comparison
// network sorted them.
__global__ __launch_bounds__(SEL_NT) void k_selftest_sort(const unsigned long long *in, int n, int cap,
                                                          unsigned long long *out, int *path) {
  extern __shared__ unsigned long long keys[];
  for (int p = threadIdx.x; p < cap; p += SEL_NT) keys[p] = p < n ? in[p] : 0ull;
  const bool placed = sort_desc_u64<SEL_NT>(keys, n, cap);
  for (int p = threadIdx.x; p < n; p += SEL_NT) out[p] = keys[p];
  if (threadIdx.x == 0) *path = placed ? 0 : 1;
}

hipError_t launch_selftest_sort(const unsigned long long *in, int n, unsigned long long *out, int *path,
                                hipStream_t st) {
  const int cap = max(64, pow2_at_least(n));
  return launch_k(k_selftest_sort, dim3(1), dim3(SEL_NT), (uint32_t)sort_lds_bytes(cap), st, in, n,
                  cap, out, path);
}

}  // namespace kvq
