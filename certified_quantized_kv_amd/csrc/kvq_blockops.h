// kvq_blockops.h -- workgroup-level building blocks shared by the selection
// and controller kernels: exclusive scan, run extraction, sort of 64-bit
// keys (bucket sort in LDS), and the per-KV-head promotion planner.
#pragma once
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

__host__ __device__ inline int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Combining the partials of a workgroup's waves (at most 16, written to LDS
// by one lane each and read after a barrier): lane k < nw of every wave
// reads partial k and a scan over the first row of 16 lanes (DPP row shifts,
// zero shifted in) does the adds, so each wave spends a few vector steps
// instead of one add per partial in every one of its lanes.  Results from
// lanes of that row (readlane: wave-uniform).  The whole wave must be active.
__device__ __forceinline__ unsigned long long row0_scan_u64(unsigned long long x) {
  x += dpp_u64<0x111, 0xf>(x);
  x += dpp_u64<0x112, 0xf>(x);
  x += dpp_u64<0x114, 0xf>(x);
  x += dpp_u64<0x118, 0xf>(x);
  return x;
}
__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long x, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
  return ((unsigned long long)hi << 32) | lo;
}
// sum of partials [0, wave) and of all nw partials
__device__ __forceinline__ void wave_partials_u64(const unsigned long long *buf, int nw, int wave,
                                                  unsigned long long &before, unsigned long long &all) {
  const int lane = threadIdx.x & 63;
  const unsigned long long x = row0_scan_u64(lane < nw ? buf[lane] : 0ull);
  all = readlane_u64(x, nw - 1);
  before = wave > 0 ? readlane_u64(x, wave - 1) : 0ull;
}
__device__ __forceinline__ int wave_partials_before_i32(const int *buf, int nw, int wave) {
  const int lane = threadIdx.x & 63;
  uint32_t x = lane < nw ? (uint32_t)buf[lane] : 0u;
  x += dpp_u32<0x111, 0xf>(x);
  x += dpp_u32<0x112, 0xf>(x);
  x += dpp_u32<0x114, 0xf>(x);
  x += dpp_u32<0x118, 0xf>(x);
  return wave > 0 ? __builtin_amdgcn_readlane((int)x, wave - 1) : 0;
}
// largest of nw non-negative partials (the others read as 0)
__device__ __forceinline__ int wave_partials_max_i32(const int *buf, int nw) {
  const int lane = threadIdx.x & 63;
  int x = lane < nw ? buf[lane] : 0;
  x = max(x, (int)dpp_u32<0x111, 0xf>((uint32_t)x));
  x = max(x, (int)dpp_u32<0x112, 0xf>((uint32_t)x));
  x = max(x, (int)dpp_u32<0x114, 0xf>((uint32_t)x));
  x = max(x, (int)dpp_u32<0x118, 0xf>((uint32_t)x));
  return __builtin_amdgcn_readlane(x, nw - 1);
}

// smallest and largest of nw u32 partials (the identities shifted in)
__device__ __forceinline__ uint32_t wave_partials_min_u32(const uint32_t *buf, int nw) {
  const int lane = threadIdx.x & 63;
  constexpr int ALL = -1;
  uint32_t x = lane < nw ? buf[lane] : 0xffffffffu;
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(ALL, (int)x, 0x111, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(ALL, (int)x, 0x112, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(ALL, (int)x, 0x114, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(ALL, (int)x, 0x118, 0xf, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, nw - 1);
}
__device__ __forceinline__ uint32_t wave_partials_max_u32(const uint32_t *buf, int nw) {
  const int lane = threadIdx.x & 63;
  uint32_t x = lane < nw ? buf[lane] : 0u;
  x = max(x, dpp_u32<0x111, 0xf>(x));
  x = max(x, dpp_u32<0x112, 0xf>(x));
  x = max(x, dpp_u32<0x114, 0xf>(x));
  x = max(x, dpp_u32<0x118, 0xf>(x));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, nw - 1);
}
// largest of nw float partials (-inf shifted in)
__device__ __forceinline__ float wave_partials_max_f32(const float *buf, int nw) {
  const int lane = threadIdx.x & 63;
  constexpr int NEG = (int)0xff800000u;   // -inf
  float x = lane < nw ? buf[lane] : -INFINITY;
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(NEG, __float_as_int(x), 0x111, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(NEG, __float_as_int(x), 0x112, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(NEG, __float_as_int(x), 0x114, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(NEG, __float_as_int(x), 0x118, 0xf, 0xf, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), nw - 1));
}

// Block-wide exclusive scan of small counts (blockDim multiple of 64); every
// thread adds up the wave totals below its own.  tmp holds blockDim / 64
// entries and is free again after the caller's next barrier.
__device__ inline int block_excl_scan(int v, int *tmp, int &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int x = (int)wave_incl_scan_u32((uint32_t)v);
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
  for (int k = 0; k < nw; ++k) {
    const int c = tmp[k];
    if (k < wave) before += c;
    all += c;
  }
  total = all;
  return before + x - v;
}

// Runs of consecutive set flags (flags[0..NB)) -> runs[k] = start | len << 16.
// Thread t scans the flags [t E, (t+1) E); one exclusive scan of its packed
// (starts | ends << 16) counts gives every start and every (exclusive) end its
// rank, so the k-th start pairs with the k-th end; the two halves of runs[k]
// are written by the threads that found them, then joined.
__device__ inline int build_runs(const uint8_t *flags, int NB, uint32_t *runs, int *tmp) {
  uint16_t *half = reinterpret_cast<uint16_t *>(runs);
  const int E = (NB + (int)blockDim.x - 1) / (int)blockDim.x;
  const int b0 = threadIdx.x * E, b1 = min(NB, b0 + E);
  int ns = 0, ne = 0;
  for (int b = b0; b < b1; ++b) {
    if (!flags[b]) continue;
    ns += (b == 0 || !flags[b - 1]) ? 1 : 0;
    ne += (b == NB - 1 || !flags[b + 1]) ? 1 : 0;
  }
  int total;
  const int pre = block_excl_scan(ns | (ne << 16), tmp, total);
  int ps = pre & 0xffff, pe = pre >> 16;
  for (int b = b0; b < b1; ++b) {
    if (!flags[b]) continue;
    if (b == 0 || !flags[b - 1]) half[2 * (ps++)] = (uint16_t)b;
    if (b == NB - 1 || !flags[b + 1]) half[2 * (pe++) + 1] = (uint16_t)(b + 1);
  }
  const int nr = total & 0xffff;
  __syncthreads();
  for (int k = threadIdx.x; k < nr; k += blockDim.x) {
    const uint32_t r = runs[k];
    const uint32_t st = r & 0xffffu, en = r >> 16;
    runs[k] = st | ((en - st) << 16);
  }
  __syncthreads();
  return nr;
}

// Plan for the host (device words, 64-bit): [0] number of K runs, [1] number
// of V runs, [2] flags (bit0: a group is still widening, bit1: some head is at
// rung 3), [3] nonzero when the first controller round flagged a head for the
// group decisions, then K entries from word 4 and V entries from word 4 + kcap, each
// len | start << 16 | ig << 32 | kind << 48 with ig = i * Hkv + g.  Groups
// reserve their entries with atomics (entry order is immaterial to the copies).
__device__ inline void emit_runs(const Shape &s, const Step &w, int ig, int kind,
                                 const uint32_t *runs, int nr, int *sbase) {
  if (threadIdx.x == 0)
    *sbase = nr ? (int)atomicAdd(&w.plan[kind], (unsigned long long)nr) : 0;
  __syncthreads();
  const size_t off = 4 + (kind ? plan_kcap(s) : 0) + (size_t)*sbase;
  for (int k = threadIdx.x; k < nr; k += blockDim.x) {
    const uint32_t r = runs[k];
    w.plan[off + k] = (unsigned long long)(r >> 16) | ((unsigned long long)(r & 0xffffu) << 16) |
                      ((unsigned long long)ig << 32) | ((unsigned long long)kind << 48);
  }
}

// ---- comparison sort (the bucket sort's fallback) ----------------------------
// Every wave sorts a chunk of 64*E keys in registers with a bitonic network
// (E consecutive keys per lane; partners closer than E in the same lane,
// the others exchanged across lanes with DPP / swizzle moves), then sorted
// runs are merged pairwise in LDS: a key's position in the merged run is its
// position in its own run plus the number of keys of the partner run ahead of
// it (binary search; the earlier run wins ties, so positions never collide),
// computed by every thread for its keys before any is written.
template <int E, int KK, int J>
__device__ __forceinline__ void bitonic_stage(unsigned long long (&v)[E], int lane) {
  if constexpr (J < E) {
#pragma unroll
    for (int k = 0; k < E; ++k) {
      if (k & J) continue;
      const bool desc = ((lane * E + k) & KK) == 0;
      const unsigned long long a = v[k], b = v[k | J];
      const bool swap = desc ? (a < b) : (a > b);
      v[k] = swap ? b : a;
      v[k | J] = swap ? a : b;
    }
  } else {
#pragma unroll
    for (int k = 0; k < E; ++k) {
      const int le = lane * E + k;
      const unsigned long long p = xor_lane_u64<J / E>(v[k]);
      const bool keep_max = ((le & J) == 0) == ((le & KK) == 0);
      v[k] = keep_max ? (v[k] > p ? v[k] : p) : (v[k] < p ? v[k] : p);
    }
  }
  if constexpr (J > 1) bitonic_stage<E, KK, J / 2>(v, lane);
}

template <int E, int KK, int CH>
__device__ __forceinline__ void bitonic_chunk(unsigned long long (&v)[E], int lane) {
  bitonic_stage<E, KK, KK / 2>(v, lane);
  if constexpr (KK < CH) bitonic_chunk<E, KK * 2, CH>(v, lane);
}

// Number of entries of the descending run a[0..len) ahead of x: those > x
// (ties = false) or >= x (ties = true).
__device__ __forceinline__ int count_ahead(const unsigned long long *a, int len,
                                           unsigned long long x, bool ties) {
  int lo = 0, hi = len;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const unsigned long long y = a[mid];
    if (y > x || (ties && y == x)) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

template <int NT, int E>
__device__ __forceinline__ void sort_desc_network(unsigned long long *keys, int n) {
  constexpr int CH = 64 * E;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = (n + CH - 1) / CH;
  const int cap = nch * CH;
  const bool active = wave < nch;
  unsigned long long v[E];
  int pos[E];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < E; ++k) {
    pos[k] = wave * CH + lane * E + k;
    v[k] = (active && pos[k] < n) ? keys[pos[k]] : 0ull;
  }
  if (active) bitonic_chunk<E, 2, CH>(v, lane);
  __syncthreads();
  if (active) {
#pragma unroll
    for (int k = 0; k < E; ++k) keys[pos[k]] = v[k];
  }
  for (int R = CH; R < cap; R <<= 1) {
    __syncthreads();
    int np[E];
    if (active) {
#pragma unroll
      for (int k = 0; k < E; ++k) {
        const int id = pos[k] / R;
        const int ps = (id ^ 1) * R;
        const int plen = max(0, min(R, cap - ps));
        const int cnt = count_ahead(keys + ps, plen, v[k], (id & 1) != 0);
        np[k] = (id & ~1) * R + (pos[k] - id * R) + cnt;
      }
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int k = 0; k < E; ++k) {
        pos[k] = np[k];
        keys[np[k]] = v[k];
      }
    }
  }
  __syncthreads();
}

// ---- block sort of distinct 64-bit keys into descending order --------------
// Bucket sort by a monotone image of each key: its binary32 image, cut into
// 4096 buckets on a log-like scale (the float bits), or, if that crowds a
// bucket, key - smallest key on a linear scale.  Each thread keeps its keys
// in registers; counting them into buckets with LDS atomics also gives each
// key a slot in its bucket.  A key alone in its bucket goes straight to its
// final place (the bucket's start); the others are scattered by slot and
// take their place inside the bucket by counting the bucket's keys ahead of
// them.  The result does not depend on the order of the atomics.  When both
// images leave more than SORT_MAX_BUCKET keys in some bucket (clusters of
// keys that differ only far below their leading bits) the comparison network
// above sorts instead.  The caller's LDS buffer `keys` holds
// sort_lds_bytes(cap) bytes (cap >= n keys, cap a power of two >= 64,
// n <= MAX_NB).
constexpr int SORT_BUCKETS = 4096;

__host__ __device__ inline size_t sort_lds_bytes(int cap) {
  return (size_t)cap * 16 + (size_t)(2 * SORT_BUCKETS + 2) * 4;
}

__device__ __forceinline__ uint32_t key_image(unsigned long long k) {
  return __float_as_uint((float)k);      // round to nearest: non-decreasing in k
}

// Buckets larger than this send the whole sort to the comparison network.
constexpr int SORT_MAX_BUCKET = 48;

// Callable on each key's final position (bucket path); the comparison
// network path does not call it and sort_desc_u64 then returns false.
struct NoPlace {
  __device__ void operator()(unsigned long long, int) const {}
};

// The sort with the keys already in the caller's registers: kv[r] is the key
// at position t + r NT of keys[0 .. n) (thread t), and keys[] holds them too
// (the comparison network reads them there), written by the caller before the
// call; the sort's own LDS (tmp, the bucket counters) is not touched by the
// caller before it, so the sort starts without a barrier.  RK = keys per
// thread: the caller guarantees n <= RK * NT.
template <int NT, int RK, class OnPlace = NoPlace>
__device__ __forceinline__ bool sort_desc_u64_regs(const unsigned long long (&kv)[RK], unsigned long long *keys,
                                                   int n, int cap, OnPlace on_place = OnPlace()) {
  constexpr int SB = SORT_BUCKETS;
  constexpr int PER = SB / NT;           // counters per thread in the scan
  static_assert(SB % NT == 0, "bucket count");
  static_assert(4 * NT >= MAX_NB, "the comparison network's chunks (4 keys per lane) cover MAX_NB keys");
  unsigned long long *tmp = keys + cap;
  int *base = reinterpret_cast<int *>(keys + 2 * (size_t)cap);   // SB + 1 entries
  int *cur = base + SB + 1;                                     // SB entries
  __shared__ unsigned long long kred[2][NT / 64];
  __shared__ uint32_t red[2][NT / 64];
  __shared__ int wsum[2][NT / 64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // image 1: the key's own binary32 image, over the images' range
  int bk[RK], slot[RK];
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int r = 0; r < RK; ++r) {
    const int p = threadIdx.x + r * NT;
    if (p < n) {
      const uint32_t f = key_image(kv[r]);
      lo = min(lo, f);
      hi = max(hi, f);
    }
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    red[0][wave] = lo;
    red[1][wave] = hi;
  }
  for (int k = threadIdx.x; k < SB; k += NT) cur[k] = 0;
  __syncthreads();
  lo = wave_partials_min_u32(red[0], NT / 64);
  hi = wave_partials_max_u32(red[1], NT / 64);
  // image 2 (used when image 1 crowds a bucket): key - smallest key on a
  // linear scale, which separates keys that agree in their leading bits
  bool rel = false;
  int sh = 0;
  unsigned long long kmin = 0ull;
  auto bucket = [&](unsigned long long k) {
    const int f = rel ? (int)((k - kmin) >> sh) : (int)((key_image(k) - lo) >> sh);
    return SB - 1 - f;
  };
  int c[PER];
  int own = 0, xs = 0, big = 0;
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 0) {
      const uint32_t span = hi - lo;
      sh = span >= (uint32_t)SB ? (32 - __clz((int)span)) - 12 : 0;
    } else {
      rel = true;
      unsigned long long kmn = ~0ull, kmx = 0ull;
#pragma unroll
      for (int r = 0; r < RK; ++r) {
        if (threadIdx.x + r * NT < n) {
          kmn = min(kmn, kv[r]);
          kmx = max(kmx, kv[r]);
        }
      }
      kmn = wave_min_u64(kmn);
      kmx = wave_max_u64(kmx);
      if (lane == 0) {
        kred[0][wave] = kmn;
        kred[1][wave] = kmx;
      }
      for (int k = threadIdx.x; k < SB; k += NT) cur[k] = 0;
      __syncthreads();
      kmin = kred[0][0];
      unsigned long long kmax = kred[1][0];
#pragma unroll
      for (int k = 1; k < NT / 64; ++k) {
        kmin = min(kmin, kred[0][k]);
        kmax = max(kmax, kred[1][k]);
      }
      const unsigned long long span = kmax - kmin;
      sh = span >= (unsigned long long)SB ? (64 - __clzll((long long)span)) - 12 : 0;
    }
#pragma unroll
    for (int r = 0; r < RK; ++r) {
      if (threadIdx.x + r * NT < n) {
        bk[r] = bucket(kv[r]);
        slot[r] = atomicAdd(&cur[bk[r]], 1);
      }
    }
    __syncthreads();
    // this thread's counters [t PER, (t+1) PER): their sum, scanned over the
    // wave, and the largest count, reduced over the wave
    own = 0;
    big = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      c[k] = cur[threadIdx.x * PER + k];
      own += c[k];
      big = max(big, c[k]);
    }
    xs = (int)wave_incl_scan_u32((uint32_t)own);
    big = (int)wave_max_u32((uint32_t)big);
    if (lane == 63) wsum[0][wave] = xs;
    if (lane == 0) wsum[1][wave] = big;
    __syncthreads();
    big = wave_partials_max_i32(wsum[1], NT / 64);
    if (big <= SORT_MAX_BUCKET) break;
    if (pass == 1) {
      // clustered keys: comparison network instead (the keys are untouched)
      if (n <= NT)
        sort_desc_network<NT, 1>(keys, n);
      else if (n <= 2 * NT)
        sort_desc_network<NT, 2>(keys, n);
      else
        sort_desc_network<NT, 4>(keys, n);
      return false;
    }
    __syncthreads();                     // wsum and cur are written again by pass 1
  }
  // exclusive prefix of the counts -> base
  const int before = wave_partials_before_i32(wsum[0], NT / 64, wave);
  int run = before + xs - own;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    base[threadIdx.x * PER + k] = run;
    run += c[k];
  }
  if (threadIdx.x == 0) base[SB] = n;
  __syncthreads();
  // a key alone in its bucket is placed; the others are scattered by slot
  int b0[RK], b1[RK];
#pragma unroll
  for (int r = 0; r < RK; ++r) {
    if (threadIdx.x + r * NT >= n) continue;
    b0[r] = base[bk[r]];
    b1[r] = base[bk[r] + 1];
    if (b1[r] - b0[r] == 1) {
      keys[b0[r]] = kv[r];
      on_place(kv[r], b0[r]);
    } else {
      tmp[b0[r] + slot[r]] = kv[r];
    }
  }
  if (big > 1) {
    __syncthreads();
    // place inside the bucket: keys ahead = larger keys (the keys are
    // distinct, so that count is the rank)
#pragma unroll
    for (int r = 0; r < RK; ++r) {
      if (threadIdx.x + r * NT >= n || b1[r] - b0[r] == 1) continue;
      const unsigned long long k = kv[r];
      int rk = 0;
      int q = b0[r];
      for (; q + 4 <= b1[r]; q += 4) {
        const unsigned long long y0 = tmp[q], y1 = tmp[q + 1], y2 = tmp[q + 2], y3 = tmp[q + 3];
        rk += (y0 > k ? 1 : 0) + (y1 > k ? 1 : 0) + (y2 > k ? 1 : 0) + (y3 > k ? 1 : 0);
      }
      for (; q < b1[r]; ++q) rk += tmp[q] > k ? 1 : 0;
      keys[b0[r] + rk] = k;
      on_place(k, b0[r] + rk);
    }
  }
  __syncthreads();
  return true;
}

// The sort of keys[0 .. n) in LDS (written by the caller before the call).
template <int NT, int RK = (MAX_NB + NT - 1) / NT, class OnPlace = NoPlace>
__device__ __forceinline__ bool sort_desc_u64(unsigned long long *keys, int n, int cap,
                                              OnPlace on_place = OnPlace()) {
  __syncthreads();
  unsigned long long kv[RK];
#pragma unroll
  for (int r = 0; r < RK; ++r) {
    const int p = threadIdx.x + r * NT;
    kv[r] = p < n ? keys[p] : 0ull;
  }
  return sort_desc_u64_regs<NT, RK>(kv, keys, n, cap, on_place);
}

// Inclusive scan of per-thread u64 values over a workgroup of NT threads
// (NT = 64 * waves); returns the inclusive prefix, total in *total.  With
// REUSE false the caller writes buf again only after a barrier of its own,
// so the scan ends without one.
template <int NT, bool REUSE = true>
__device__ inline unsigned long long block_incl_scan_u64(unsigned long long v, unsigned long long *buf,
                                                         unsigned long long *total) {
  static_assert(NT / 64 <= 16, "one partial per lane of a row");
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const unsigned long long x = wave_incl_scan_u64(v);
  if (lane == 63) buf[wave] = x;
  __syncthreads();
  unsigned long long before, all;
  wave_partials_u64(buf, NT / 64, wave, before, all);
  if (REUSE) __syncthreads();
  *total = all;
  return x + before;
}

// Union of the group's selections -> U; blocks new to U -> Knew and K runs.
// Flags live in LDS while the group is planned; U and Knew are written back.
__device__ inline void plan_group_keys(const Shape &s, const Step &w, int i, int g, int NB) {
  __shared__ int tmp[18];
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
  emit_runs(s, w, i * s.Hkv + g, 0, runs, nr, tmp + 17);
}

// Step set-up, spread over the threads of the first kernel of a step (nt
// threads, this one numbered tid): q' = fl32(q * C) (log2 units) for the n
// call positions, and the per-step flags and head state cleared (byte arrays
// [n][Hkv][NBmax] and [n][Hq][NBmax], head/group words, plan headers).
__device__ inline void step_setup(const Shape &s, const Step &w, int n, const uint16_t *q, float C,
                                  size_t tid, size_t nt) {
  const size_t nb_g = (size_t)n * s.Hkv * s.NBmax, nb_h = (size_t)n * s.Hq * s.NBmax;
  for (size_t k = tid; k < (size_t)n * s.Hq * s.d; k += nt) w.qp[k] = h2f(q[k]) * C;
  for (size_t k = tid; k < nb_g; k += nt) {
    w.U[k] = 0;
    w.Knew[k] = 0;
    w.V[k] = 0;
  }
  for (size_t k = tid; k < nb_h; k += nt) w.vh[k] = 0;
  for (size_t k = tid; k < (size_t)n * s.Hq; k += nt) {
    w.hflags[k] = 0u;
    w.ekey64[k] = 0.0;
    w.eval64[k] = 0.0;
  }
  for (size_t k = tid; k < (size_t)n * s.Hkv; k += nt) w.gstat[k] = 0u;
  if (tid < 4) w.plan[tid] = 0ull;
}

}  // namespace kvq
