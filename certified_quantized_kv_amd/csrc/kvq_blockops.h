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

// ---- block sort of distinct 64-bit keys into descending order -------------
// Bitonic network on a power-of-two count n2 (64 <= n2 <= 16 * NT).  Each
// thread keeps E = max(1, n2/NT) consecutive keys in registers: partners
// closer than E are in the same thread, partners closer than 64*E in the same
// wave (exchanged with compile-time lane masks), and only the wider stages go
// through LDS with barriers.
__device__ __forceinline__ unsigned long long cx_pick(unsigned long long a, unsigned long long b,
                                                      bool keep_max) {
  return keep_max ? (a > b ? a : b) : (a < b ? a : b);
}

template <int E, int LJ>
__device__ __forceinline__ void inwave_stage(unsigned long long (&v)[E], int t, int kk) {
  constexpr int J = LJ * E;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const int e = t * E + k;
    const unsigned long long p = __shfl_xor(v[k], LJ, 64);
    v[k] = cx_pick(v[k], p, ((e & J) == 0) == ((e & kk) == 0));
  }
}

template <int E, int JJ>
__device__ __forceinline__ void inthread_stage(unsigned long long (&v)[E], int t, int kk) {
#pragma unroll
  for (int k = 0; k < E; ++k) {
    if (k & JJ) continue;
    const int e = t * E + k;
    const unsigned long long a = v[k], b = v[k | JJ];
    const bool desc = (e & kk) == 0;
    if (desc ? (a < b) : (a > b)) {
      v[k] = b;
      v[k | JJ] = a;
    }
  }
}

template <int NT, int E>
__device__ inline void sort_desc_pow2_e(unsigned long long *keys, int n2) {
  const int act = n2 / E;
  const int t = threadIdx.x;
  unsigned long long v[E];
#pragma unroll
  for (int k = 0; k < E; ++k) v[k] = 0ull;
  __syncthreads();
  if (t < act) {
#pragma unroll
    for (int k = 0; k < E; ++k) v[k] = keys[t * E + k];
  }
  for (int kk = 2; kk <= n2; kk <<= 1) {
    // stages whose partner lives in another wave: through LDS
    for (int j = kk >> 1; j >= 64 * E; j >>= 1) {
      __syncthreads();
      if (t < act) {
#pragma unroll
        for (int k = 0; k < E; ++k) keys[t * E + k] = v[k];
      }
      __syncthreads();
      if (t < act) {
#pragma unroll
        for (int k = 0; k < E; ++k) {
          const int e = t * E + k;
          v[k] = cx_pick(v[k], keys[e ^ j], ((e & j) == 0) == ((e & kk) == 0));
        }
      }
    }
    // stages within a wave, then within a thread (partner distance j = LJ*E)
    const int top = kk >> 1;
    if (top >= 32 * E) inwave_stage<E, 32>(v, t, kk);
    if (top >= 16 * E) inwave_stage<E, 16>(v, t, kk);
    if (top >= 8 * E) inwave_stage<E, 8>(v, t, kk);
    if (top >= 4 * E) inwave_stage<E, 4>(v, t, kk);
    if (top >= 2 * E) inwave_stage<E, 2>(v, t, kk);
    if (top >= E) inwave_stage<E, 1>(v, t, kk);
    if (E >= 16 && top >= 8) inthread_stage<E, (E >= 16 ? 8 : 1)>(v, t, kk);
    if (E >= 8 && top >= 4) inthread_stage<E, (E >= 8 ? 4 : 1)>(v, t, kk);
    if (E >= 4 && top >= 2) inthread_stage<E, (E >= 4 ? 2 : 1)>(v, t, kk);
    if (E >= 2 && top >= 1) inthread_stage<E, 1>(v, t, kk);
  }
  __syncthreads();
  if (t < act) {
#pragma unroll
    for (int k = 0; k < E; ++k) keys[t * E + k] = v[k];
  }
  __syncthreads();
}

template <int NT>
__device__ inline void sort_desc_pow2(unsigned long long *keys, int n2) {
  if (n2 <= NT)
    sort_desc_pow2_e<NT, 1>(keys, n2);
  else if (n2 <= 2 * NT)
    sort_desc_pow2_e<NT, 2>(keys, n2);
  else if (n2 <= 4 * NT)
    sort_desc_pow2_e<NT, 4>(keys, n2);
  else if (n2 <= 8 * NT)
    sort_desc_pow2_e<NT, 8>(keys, n2);
  else
    sort_desc_pow2_e<NT, 16>(keys, n2);
}

// Sorts n distinct keys keys[0..n) into descending order (n <= 4 * NT); the
// buffer must hold pow2(n) entries.  n = A + B with A the largest power of two
// <= n (at least 64): A and B (zero-padded to a power of two) are sorted by
// the network above and merged in place: every key's output position is found
// by binary search in the other run (keys are distinct, so positions never
// collide), kept in registers, and written after a barrier.
template <int NT>
__device__ inline void sort_desc_u64(unsigned long long *keys, int n) {
  int A = 64;
  while (A * 2 <= n) A <<= 1;
  if (n <= A) {
    for (int k = n + threadIdx.x; k < A; k += NT) keys[k] = 0ull;
    sort_desc_pow2<NT>(keys, A);
    return;
  }
  const int B = n - A;
  int B2 = 64;
  while (B2 < B) B2 <<= 1;
  unsigned long long *kb = keys + A;
  for (int k = B + threadIdx.x; k < B2; k += NT) kb[k] = 0ull;
  sort_desc_pow2<NT>(keys, A);
  sort_desc_pow2<NT>(kb, B2);
  unsigned long long kv[4];
  int pos[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int x = threadIdx.x + r * NT;
    pos[r] = -1;
    kv[r] = 0ull;
    if (x < A + B) {
      const bool inA = x < A;
      const int idx = inA ? x : x - A;
      const unsigned long long key = inA ? keys[idx] : kb[idx];
      const unsigned long long *other = inA ? kb : keys;
      int lo = 0, hi = inA ? B : A;             // count of other keys > key
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (other[mid] > key) lo = mid + 1; else hi = mid;
      }
      kv[r] = key;
      pos[r] = idx + lo;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (pos[r] >= 0) keys[pos[r]] = kv[r];
  __syncthreads();
}

// Inclusive scan of per-thread u64 values over a workgroup of NT threads
// (NT = 64 * waves); returns the inclusive prefix, total in *total.
template <int NT>
__device__ inline unsigned long long block_incl_scan_u64(unsigned long long v, unsigned long long *buf,
                                                         unsigned long long *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) buf[wave] = x;
  __syncthreads();
  unsigned long long before = 0ull, all = 0ull;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    const unsigned long long c = buf[k];
    if (k < wave) before += c;
    all += c;
  }
  __syncthreads();
  *total = all;
  return x + before;
}

// Union of the group's selections -> U; blocks new to U -> Knew and K runs.
// Flags live in LDS while the group is planned; U and Knew are written back.
__device__ inline void plan_group_keys(const Shape &s, const Step &w, int i, int g, int NB) {
  __shared__ int tmp[17];
  __shared__ uint8_t fu[MAX_NB];
  __shared__ uint8_t fk[MAX_NB];
  uint8_t *U = w.U + ((size_t)i * s.Hkv + g) * s.NBmax;
  uint8_t *Kn = w.Knew + ((size_t)i * s.Hkv + g) * s.NBmax;
  for (int b = threadIdx.x; b < NB; b += blockDim.x) {
    fu[b] = U[b];
    fk[b] = 0;
  }
  __syncthreads();
  for (int hh = 0; hh < s.G; ++hh) {
    const int hq = g * s.G + hh;
    const int ss = w.ssize[(size_t)i * s.Hq + hq];
    const uint32_t *pi = w.pi + ((size_t)i * s.Hq + hq) * s.NBmax;
    for (int k = threadIdx.x; k < ss; k += blockDim.x) {
      const uint32_t b = pi[k];
      if (!fu[b]) fk[b] = 1;     // benign race: every writer stores 1
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < NB; b += blockDim.x) {
    if (fk[b]) {
      U[b] = 1;
      Kn[b] = 1;
    }
  }
  uint32_t *runs = w.runs + (((size_t)i * s.Hkv + g) * 2 + 0) * s.runmax;
  const int nr = build_runs(fk, NB, runs, tmp);
  if (threadIdx.x == 0) w.nruns[((size_t)i * s.Hkv + g) * 2 + 0] = (uint32_t)nr;
}

}  // namespace kvq
