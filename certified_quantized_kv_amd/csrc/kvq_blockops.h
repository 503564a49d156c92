// kvq_blockops.h -- workgroup-level building blocks shared by the selection
// and controller kernels: exclusive scan, run extraction, bitonic sort of
// 64-bit keys in LDS, and the per-KV-head promotion planner.
#pragma once
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

__host__ __device__ inline int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Block-wide exclusive scan of small counts (blockDim multiple of 64).
__device__ inline int block_excl_scan(int v, int *tmp, int &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int k = 0; k < nw; ++k) {
      const int c = tmp[k];
      tmp[k] = acc;
      acc += c;
    }
    tmp[nw] = acc;
  }
  __syncthreads();
  const int r = x - v + tmp[wave];
  total = tmp[nw];
  __syncthreads();
  return r;
}

// Runs of consecutive set flags (flags[0..NB)) -> runs[k] = start | len << 16.
// Starts and (exclusive) ends are compacted separately, in increasing order,
// so the k-th start pairs with the k-th end; the two halves of runs[k] are
// written by different threads, then joined.
__device__ inline int build_runs(const uint8_t *flags, int NB, uint32_t *runs, int *tmp) {
  uint16_t *half = reinterpret_cast<uint16_t *>(runs);
  int base_s = 0, base_e = 0;
  for (int c0 = 0; c0 < NB; c0 += blockDim.x) {
    const int b = c0 + threadIdx.x;
    const bool on = b < NB && flags[b];
    const bool start = on && (b == 0 || !flags[b - 1]);
    const bool end = on && (b == NB - 1 || !flags[b + 1]);
    int ts, te;
    const int ps = block_excl_scan(start ? 1 : 0, tmp, ts);
    const int pe = block_excl_scan(end ? 1 : 0, tmp, te);
    if (start) half[2 * (base_s + ps)] = (uint16_t)b;
    if (end) half[2 * (base_e + pe) + 1] = (uint16_t)(b + 1);
    base_s += ts;
    base_e += te;
  }
  __syncthreads();
  for (int k = threadIdx.x; k < base_s; k += blockDim.x) {
    const uint32_t r = runs[k];
    const uint32_t st = r & 0xffffu, en = r >> 16;
    runs[k] = st | ((en - st) << 16);
  }
  __syncthreads();
  return base_s;
}

template <int NT>
__device__ inline void bitonic_desc(unsigned long long *keys, int n2) {
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int idx = threadIdx.x; idx < n2; idx += NT) {
        const int ixj = idx ^ j;
        if (ixj > idx) {
          const unsigned long long a = keys[idx], b = keys[ixj];
          const bool desc = (idx & k) == 0;
          if (desc ? (a < b) : (a > b)) {
            keys[idx] = b;
            keys[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Union of the group's selections -> U; blocks new to U -> Knew and K runs.
__device__ inline void plan_group_keys(const Shape &s, const Step &w, int i, int g, int NB) {
  __shared__ int tmp[17];
  uint8_t *U = w.U + ((size_t)i * s.Hkv + g) * s.NBmax;
  uint8_t *Kn = w.Knew + ((size_t)i * s.Hkv + g) * s.NBmax;
  for (int hh = 0; hh < s.G; ++hh) {
    const int hq = g * s.G + hh;
    const int ss = w.ssize[(size_t)i * s.Hq + hq];
    const uint32_t *pi = w.pi + ((size_t)i * s.Hq + hq) * s.NBmax;
    for (int k = threadIdx.x; k < ss; k += blockDim.x) {
      const uint32_t b = pi[k];
      if (!U[b]) Kn[b] = 1;     // benign race: every writer stores 1
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < NB; b += blockDim.x)
    if (Kn[b]) U[b] = 1;
  __syncthreads();
  uint32_t *runs = w.runs + (((size_t)i * s.Hkv + g) * 2 + 0) * s.runmax;
  const int nr = build_runs(Kn, NB, runs, tmp);
  if (threadIdx.x == 0) w.nruns[((size_t)i * s.Hkv + g) * 2 + 0] = (uint32_t)nr;
}

}  // namespace kvq
