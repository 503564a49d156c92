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
// Promotion is per KV head: U_g = union of the group's top-K* sets; blocks
// new to U_g are listed as runs of consecutive blocks for the host copies.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_blockops.h"

namespace kvq {

constexpr int SEL_NT = 1024;

__global__ __launch_bounds__(SEL_NT) void k_select(Shape s, Step w, SeqTab tab, int tau_ppm) {
  extern __shared__ unsigned long long keys[];
  __shared__ float red[SEL_NT / 64];
  __shared__ unsigned long long sbuf[SEL_NT / 64];
  const int i = blockIdx.y, hq = blockIdx.x;
  const int T = tab.T[i], NB = (T + BLOCK - 1) / BLOCK;
  const int n2 = max(64, pow2_at_least(NB));
  const size_t base = ((size_t)i * s.Hq + hq) * s.NBmax;

  float m = -INFINITY;
  for (int b = threadIdx.x; b < NB; b += SEL_NT) m = fmaxf(m, w.mhat[base + b]);
  m = bfly_max<64>(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int k = 1; k < SEL_NT / 64; ++k) M = fmaxf(M, red[k]);

  for (int b = threadIdx.x; b < n2; b += SEL_NT) {
    unsigned long long key = 0ull;
    if (b < NB) {
      const uint32_t W = (uint32_t)floorf((float)w.Lhat[base + b] * exp2k(w.mhat[base + b] - M));
      w.What[base + b] = W;
      key = ((unsigned long long)W << 32) | (unsigned long long)(0xffffffffu - (uint32_t)b);
    }
    keys[b] = key;
  }
  sort_desc_u64<SEL_NT>(keys, NB, n2);

  // pi, then prefix sums of the sorted weights: thread t owns positions
  // [t*per, (t+1)*per)
  const int per = (n2 + SEL_NT - 1) / SEL_NT;
  const int p0 = threadIdx.x * per;
  unsigned long long own = 0ull;
  for (int k = 0; k < per; ++k) {
    const int p = p0 + k;
    if (p < NB) {
      const unsigned long long key = keys[p];
      w.pi[base + p] = 0xffffffffu - (uint32_t)(key & 0xffffffffull);
      own += key >> 32;
    }
  }
  unsigned long long total;
  const unsigned long long incl = block_incl_scan_u64<SEL_NT>(own, sbuf, &total);
  const unsigned long long need = (unsigned long long)tau_ppm * total;
  unsigned long long pre = incl - own;
  for (int k = 0; k < per; ++k) {
    const int p = p0 + k;                       // K* candidate p + 1
    if (p >= NB) break;
    const bool ok_prev = (p == 0) ? false : (1000000ull * pre >= need);
    pre += keys[p] >> 32;
    const bool ok = 1000000ull * pre >= need;
    if (ok && !ok_prev) {
      w.k0[(size_t)i * s.Hq + hq] = p + 1;
      w.ssize[(size_t)i * s.Hq + hq] = p + 1;
    }
  }
}

hipError_t launch_select(const Shape &s, const Step &w, const SeqTab &tab, int tau_ppm, int maxNB,
                         hipStream_t st) {
  const int n2 = max(64, pow2_at_least(maxNB));
  return launch_k(k_select, dim3(s.Hq, tab.n), dim3(SEL_NT), (uint32_t)sort_lds_bytes(n2), st, s,
                  w, tab, tau_ppm);
}

__global__ __launch_bounds__(1024) void k_plan_keys(Shape s, Step w, SeqTab tab) {
  const int i = blockIdx.y, g = blockIdx.x;
  const int NB = (tab.T[i] + BLOCK - 1) / BLOCK;
  plan_group_keys(s, w, i, g, NB);
}

hipError_t launch_plan_keys(const Shape &s, const Step &w, const SeqTab &tab, int maxNB,
                            hipStream_t st) {
  (void)maxNB;
  return launch_k(k_plan_keys, dim3(s.Hkv, tab.n), dim3(1024), 0, st, s, w, tab);
}

// Step set-up in one launch: q' = fl32(q * C) (log2 units) for the n call
// positions, and the per-step flags and head state cleared (byte arrays
// [n][Hkv][NBmax] and [n][Hq][NBmax], head/group words, plan header).
__global__ void k_reset(Shape s, Step w, int n, const uint16_t *__restrict__ q, float C) {
  const size_t nb_g = (size_t)n * s.Hkv * s.NBmax, nb_h = (size_t)n * s.Hq * s.NBmax;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t k = blockIdx.x * (size_t)blockDim.x + threadIdx.x; k < (size_t)n * s.Hq * s.d;
       k += stride)
    w.qp[k] = h2f(q[k]) * C;
  for (size_t k = blockIdx.x * (size_t)blockDim.x + threadIdx.x; k < nb_g; k += stride) {
    w.U[k] = 0;
    w.Knew[k] = 0;
    w.V[k] = 0;
  }
  for (size_t k = blockIdx.x * (size_t)blockDim.x + threadIdx.x; k < nb_h; k += stride) w.vh[k] = 0;
  for (size_t k = blockIdx.x * (size_t)blockDim.x + threadIdx.x; k < (size_t)n * s.Hq; k += stride) {
    w.hflags[k] = 0u;
    w.ekey64[k] = 0.0;
    w.eval64[k] = 0.0;
  }
  for (size_t k = blockIdx.x * (size_t)blockDim.x + threadIdx.x; k < (size_t)n * s.Hkv; k += stride)
    w.gstat[k] = 0u;
  if (blockIdx.x == 0 && threadIdx.x < 4) w.plan[threadIdx.x] = 0ull;
}

hipError_t launch_reset(const Shape &s, const Step &w, int n, const uint16_t *q, float C,
                        hipStream_t st) {
  return launch_k(k_reset, dim3(64), dim3(256), 0, st, s, w, n, q, C);
}


}  // namespace kvq
