// kvq_control.hip -- ranking-consistency check, the two bounds and the
// fallback ladder ("Runtime-Certified Bounded-Error Quantized Attention":
// Méthodologie §2 for E_key / E_val, Méthodologie §3 for the ranking check
// and the four rungs, Contributions clés for deterministic recovery).
//
// One workgroup per (sequence, KV head) runs one controller round for the
// group's query heads.  Readings (the page names the rungs, not triggers):
//   * ranking check: Spearman correlation between the INT8 order of the
//     promoted set S_h (positions in pi) and its FP16 order (W16 descending,
//     index ascending) must reach rho_min:
//       6e6 * sum d^2 <= (1e6 - rho_ppm) * n (n^2 - 1)     (exact integers);
//   * E_key, bound on TV(p_dense, p_used) with tail T = blocks outside U_g:
//       W+ = (Wt + 65)(1 + 2^-12), W- = Wt (1 - 2^-12)          (fp64, exact)
//       g+ = fl32(exp2k(D') - 1)(1 + 2^-16) + 2^-20, g- = fl32(1 - exp2k(-D'))(...)
//       E_key = min(1, sum_T ceil(W+ g+) / (sum_b floor(W-) - sum_T ceil(W+ g-)))
//     (1 if a tail block has D' > 20 or the denominator is <= 0);
//   * E_val = sum_{b not in V_g} ceil(W+ eta_b) / sum_b floor(W-);
//   * rung 1: a consistent head with E_key > eps_key doubles |S_h| along pi
//     while rounds remain; rung 3: ranking failure, or E_key > eps_key after
//     the last round; rung 2: a head with E_val > v_tol promotes the values of
//     blocks by contribution ceil(W+ eta_b) (descending, index ascending)
//     until E_val <= v_tol; V_g = union of the heads' choices;
//   * rung 4 (k_finalize): more than layer_frac of a sequence's heads at rung 3;
//   * FP16-values ablation (flag): V_g = every block, no rung 2, E_val = 0.
// Every sum is an integer, so no reduction order can change a decision.
#include <algorithm>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_blockops.h"
#include "kvq_mixed.h"
#include "kvq_rescore.h"

namespace kvq {


constexpr int CTL_NT = 1024;
// the evaluation's per-thread sums in LDS, six per thread (its dynamic LDS
// holds at least this much)
constexpr size_t EVAL_TOT_BYTES = 6 * CTL_NT * sizeof(unsigned long long);
constexpr double W_UP = 1.0 + 0x1p-12;
constexpr double W_DN = 1.0 - 0x1p-12;

struct CtlShared {
  unsigned long long u64[3][CTL_NT / 64];
  float f32[CTL_NT / 64];
  int i32[CTL_NT / 64];
  int flag;
  int wid;
};

__device__ int block_min_i32(int v, int *buf) {
  v = wave_min_i32(v);
  if ((threadIdx.x & 63) == 0) buf[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = buf[0];
  for (int k = 1; k < (int)(blockDim.x >> 6); ++k) r = min(r, buf[k]);
  __syncthreads();
  return r;
}

// Sums 8 u64 values per thread over the workgroup (result in every thread).
__device__ void block_sum_u64_8(unsigned long long (&v)[8], CtlShared &sh) {
  __shared__ unsigned long long buf[CTL_NT / 64][8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    v[k] = wave_sum_u64(v[k]);
  }
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int k = 0; k < 8; ++k) buf[threadIdx.x >> 6][k] = v[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    unsigned long long r = 0ull;
    for (int q = 0; q < CTL_NT / 64; ++q) r += buf[q][k];
    v[k] = r;
  }
  __syncthreads();
  (void)sh;
}

// Evaluates one head on the current U: mixed weights Wt, FP16 weights W16
// over S_h, ranking verdict and E_key.  Passes over the blocks: S_h
// membership (positions in pi), both references (mixed maximum, FP16 maximum
// over S_h), then weights, E_key sums and sort keys together.  gsp / hfp
// point at the group's and the head's state: they are read with the block
// arrays, and a final group or a head at rung 3 is not evaluated.
template <int EB>
__device__ void evaluate_head(const Shape &s, const Step &w, const Thresh &th, int i, int g, int hq,
                              int NB, const float *eta, const uint32_t *gsp, const uint32_t *hfp,
                              unsigned long long *keys, uint16_t *pos, CtlShared &sh) {
  const size_t base = ((size_t)i * s.Hq + hq) * s.NBmax;
  const uint8_t *U = w.U + ((size_t)i * s.Hkv + g) * s.NBmax;
  const int n = w.ssize[(size_t)i * s.Hq + hq];
  const uint32_t *pi = w.pi + base;
  __shared__ float mred[2][CTL_NT / 64];
  __shared__ unsigned long long sred[6][CTL_NT / 64];
  // every per-block input of this thread's blocks b = t + r CTL_NT (EB of
  // them) is loaded once, up front (both score kinds; the block's kind
  // selects afterwards), so the passes below wait on no global load
  const uint32_t gsv = *gsp, hfv = *hfp;
  bool pr[EB];
  float mb[EB], dl[EB], et[EB];
  uint32_t Lb[EB], pk[EB];
#pragma unroll
  for (int r = 0; r < EB; ++r) {
    const int b = threadIdx.x + r * CTL_NT;
    if (b < NB) {
      const float m16 = w.m16[base + b], mh = w.mhat[base + b];
      const uint32_t l16 = w.L16[base + b], lh = w.Lhat[base + b];
      pr[r] = U[b] != 0;
      mb[r] = pr[r] ? m16 : mh;
      Lb[r] = pr[r] ? l16 : lh;
      dl[r] = w.delta[base + b];
      et[r] = eta[b];
      pk[r] = pi[b];                    // the block at INT8 position b
    }
  }
  if ((gsv & 1u) || (hfv & 4u)) return;   // the whole workgroup leaves
  // S_h = pi[0 .. n): INT8 position of each member, 0xffff elsewhere (pi is
  // a permutation of the blocks, so one scatter writes every entry)
#pragma unroll
  for (int r = 0; r < EB; ++r) {
    const int k = threadIdx.x + r * CTL_NT;
    if (k < NB) pos[pk[r]] = k < n ? (uint16_t)k : (uint16_t)0xffff;
  }
  __syncthreads();
  // references: Mt over the mixed block maxima, M16 over S_h (S_h lies in U)
  float mloc = -INFINITY, m16loc = -INFINITY;
#pragma unroll
  for (int r = 0; r < EB; ++r) {
    const int b = threadIdx.x + r * CTL_NT;
    if (b < NB) {
      mloc = fmaxf(mloc, mb[r]);
      if (pos[b] != 0xffff) m16loc = fmaxf(m16loc, mb[r]);
    }
  }
  mloc = bfly_max<64>(mloc);
  m16loc = bfly_max<64>(m16loc);
  if ((threadIdx.x & 63) == 0) {
    mred[0][threadIdx.x >> 6] = mloc;
    mred[1][threadIdx.x >> 6] = m16loc;
  }
  __syncthreads();
  const float Mt = wave_partials_max_f32(mred[0], CTL_NT / 64);
  const float M16 = wave_partials_max_f32(mred[1], CTL_NT / 64);
  // mixed weights, E_key sums and the E_val numerator with no value
  // promoted; FP16 weights and sort keys of S_h
  unsigned long long den = 0ull, num = 0ull, sub = 0ull, cap = 0ull, numv = 0ull;
#pragma unroll
  for (int r = 0; r < EB; ++r) {
    const int b = threadIdx.x + r * CTL_NT;
    if (b >= NB) continue;
    const uint32_t Wt = (uint32_t)floorf((float)Lb[r] * exp2k(mb[r] - Mt));
    w.Wt[base + b] = Wt;
    const double Wp = (double)(Wt + 65u) * W_UP;
    const double Wm = (double)Wt * W_DN;
    den += (unsigned long long)floor(Wm);
    numv += (unsigned long long)ceil(Wp * (double)et[r]);
    if (!pr[r]) {
      if (dl[r] > 20.0f) {
        cap = 1ull;
      } else {
        const float up = exp2k(dl[r]) - 1.0f;
        const float dn = 1.0f - exp2k(-dl[r]);
        const double gp = (double)up * (1.0 + 0x1p-16) + 0x1p-20;
        const double gm = (double)dn * (1.0 + 0x1p-16) + 0x1p-20;
        num += (unsigned long long)ceil(Wp * gp);
        sub += (unsigned long long)ceil(Wp * gm);
      }
    }
    uint32_t W16 = 0u;
    const int pb = pos[b];
    if (pb != 0xffff) {
      W16 = (uint32_t)floorf((float)Lb[r] * exp2k(mb[r] - M16));
      keys[pb] = ((unsigned long long)W16 << 32) | (unsigned long long)(0xffffffffu - (uint32_t)b);
    }
    w.W16[base + b] = W16;
  }
  // ranking over S_h: FP16 order (W16 descending, index ascending); each
  // member's squared rank difference is taken where the sort places it
  const int n2 = max(64, pow2_at_least(n));
  unsigned long long ssd = 0ull;
  const bool placed = sort_desc_u64<CTL_NT, EB>(keys, n, n2, [&](unsigned long long k, int j) {
    const uint32_t b = 0xffffffffu - (uint32_t)(k & 0xffffffffull);
    const long long dd = (long long)pos[b] - (long long)j;
    ssd += (unsigned long long)(dd * dd);
  });
  if (!placed) {
    for (int j = threadIdx.x; j < n; j += CTL_NT) {
      const uint32_t b = 0xffffffffu - (uint32_t)(keys[j] & 0xffffffffull);
      const long long dd = (long long)pos[b] - (long long)j;
      ssd += (unsigned long long)(dd * dd);
    }
    __syncthreads();                      // keys[] is read; its LDS is reused below
  }
  // one reduction for the E_key sums, the E_val numerator and the ranks:
  // every thread's six sums go through LDS (the sort's area, free again),
  // wave k < 6 adds quantity k over the threads, thread 0 takes the totals
  // (integers: exact in any order; far fewer cross-lane steps than six
  // reductions in each of the sixteen waves)
  unsigned long long *tot = keys;         // [6][CTL_NT]
  {
    const unsigned long long v[6] = {den, num, sub, cap, numv, ssd};
#pragma unroll
    for (int k = 0; k < 6; ++k) tot[k * CTL_NT + threadIdx.x] = v[k];
  }
  __syncthreads();
  {
    const int wv = threadIdx.x >> 6, ln = threadIdx.x & 63;
    if (wv < 6) {
      unsigned long long r = 0ull;
#pragma unroll
      for (int j = 0; j < CTL_NT / 64; ++j) r += tot[wv * CTL_NT + ln + 64 * j];
      r = wave_sum_u64(r);
      if (ln == 0) sred[wv][0] = r;
    }
  }
  __syncthreads();
  unsigned long long v4[6];
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 0; k < 6; ++k) v4[k] = sred[k][0];
    double ek;
    if (v4[3]) {
      ek = 1.0;
    } else {
      const long long D = (long long)v4[0] - (long long)v4[2];
      ek = (D <= 0) ? 1.0 : fmin(1.0, (double)v4[1] / (double)D);
    }
    ssd = v4[5];
    const unsigned long long nn = (unsigned long long)n;
    const bool ok = (n <= 1) ||
                    (6000000ull * ssd <= (unsigned long long)(1000000 - th.rho_ppm) * nn * (nn * nn - 1ull));
    w.ssd[(size_t)i * s.Hq + hq] = ssd;
    w.ekey64[(size_t)i * s.Hq + hq] = ek;
    w.evs[2 * ((size_t)i * s.Hq + hq)] = v4[4];
    w.evs[2 * ((size_t)i * s.Hq + hq) + 1] = v4[0];
    uint32_t f = hfv;                   // written by this workgroup only
    f = ok ? (f | 1u) : ((f & ~1u) | 4u);
    w.hflags[(size_t)i * s.Hq + hq] = f;
    // a head the group decisions would act on: a ranking failure (rung 3),
    // E_key above eps_key (rung 1 or 3) or E_val above v_tol (rung 2).  When
    // no head of the first round is flagged, the decisions are known without
    // the group pass: level 0, E_val from these sums (see k_combine)
    const bool acts = !ok || ek > th.eps_key || (double)v4[4] / (double)v4[0] > th.v_tol;
    if (acts) atomicOr(&w.plan[3], 1ull);
  }
}

// Rung 2 for one head with E_val(no value promoted) = numv / denv > v_tol:
// greedy value promotion by contribution; sets vh / V flags.
__device__ void value_rung(const Shape &s, const Tier1 &t, const Step &w, const Thresh &th, int i,
                           int g, int hq, int NB, size_t unit, unsigned long long numv,
                           unsigned long long denv, unsigned long long *keys, CtlShared &sh) {
  const size_t base = ((size_t)i * s.Hq + hq) * s.NBmax;
  const float *eta = t.eta + unit * s.NBmax;
  const int n2 = max(64, pow2_at_least(NB));
  for (int b = threadIdx.x; b < n2; b += CTL_NT) {
    unsigned long long key = 0ull;
    if (b < NB) {
      const uint32_t Wt = w.Wt[base + b];
      const unsigned long long c =
          (unsigned long long)ceil((double)(Wt + 65u) * W_UP * (double)eta[b]);
      key = (c << 12) | (unsigned long long)(4095 - b);
    }
    keys[b] = key;
  }
  __syncthreads();
  sort_desc_u64<CTL_NT>(keys, NB, n2);
  // prefix sums of the sorted contributions: thread t owns [t*per, (t+1)*per)
  const int per = (NB + CTL_NT - 1) / CTL_NT;
  const int p0 = threadIdx.x * per;
  unsigned long long own = 0ull;
  for (int k = 0; k < per; ++k)
    if (p0 + k < NB) own += keys[p0 + k] >> 12;
  unsigned long long total;
  const unsigned long long incl = block_incl_scan_u64<CTL_NT>(own, sh.u64[0], &total);
  unsigned long long pre = incl - own;
  int kmin = NB;
  for (int k = 0; k < per; ++k) {
    const int p = p0 + k;
    if (p >= NB) break;
    pre += keys[p] >> 12;
    const unsigned long long rem = numv - pre;
    if ((double)rem / (double)denv <= th.v_tol) {
      kmin = p + 1;
      break;
    }
  }
  kmin = block_min_i32(kmin, sh.i32);
  uint8_t *vh = w.vh + base;
  uint8_t *V = w.V + ((size_t)i * s.Hkv + g) * s.NBmax;
  for (int p = threadIdx.x; p < kmin; p += CTL_NT) {
    const int b = 4095 - (int)(keys[p] & 4095ull);
    vh[b] = 1;
    V[b] = 1;   // benign race across heads: every writer stores 1
  }
  __syncthreads();
}

// One controller round, part 1: every query head not yet at rung 3, in a
// group not yet final, is evaluated on the group's current U (one workgroup
// per query head).
template <int EB>
__device__ inline void eval_wg(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab,
                               int layer, const Thresh &th, int i, int hq, unsigned long long *keys,
                               uint16_t *pos, CtlShared &sh) {
  const int g = hq / s.G;
  // a new plan starts with this round (the host has read the previous one);
  // word 3 (heads flagged for the group decisions) is cleared at the start of
  // the step and only read after the first round
  if (i == 0 && hq == 0 && threadIdx.x < 3) w.plan[threadIdx.x] = 0ull;
  const int NB = (tab.T[i] + BLOCK - 1) / BLOCK;
  const float *eta = t.eta + unit_of(s, tab.slot[i], layer, g) * s.NBmax;
  evaluate_head<EB>(s, w, th, i, g, hq, NB, eta, w.gstat + (size_t)i * s.Hkv + g,
                    w.hflags + (size_t)i * s.Hq + hq, keys, pos, sh);
}

// Grid (Hq + R, n): the heads, then (sequence slot 0 only) R workgroups that
// compute the INT8 scores of rlist's blocks outside U for a step whose
// scoring pass stored none, one wave per block.  Nothing in the round reads
// them, and these short-lived workgroups run beside the heads' longer chains
// of phases.
template <int EB>
__global__ __launch_bounds__(CTL_NT) void k_eval(Shape s, Tier1 t, Step w, SeqTab tab, int layer,
                                                 Thresh th, const uint16_t *q16, float C,
                                                 const uint32_t *rlist, int rcount) {
  extern __shared__ __align__(16) unsigned long long keys[];
  __shared__ uint16_t pos[MAX_NB];
  __shared__ CtlShared sh;
  if ((int)blockIdx.x >= s.Hq) {
    if (blockIdx.y != 0) return;
    constexpr int NWV = CTL_NT / 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int k0 = ((int)blockIdx.x - s.Hq) * NWV + wave, ks = ((int)gridDim.x - s.Hq) * NWV;
    if (s.d == 128)
      rescore_units<128>(s, t, w, tab, layer, q16, C, rlist, rcount, k0, ks,
                         reinterpret_cast<RescoreLds<128> *>(keys)[wave]);
    else
      rescore_units<64>(s, t, w, tab, layer, q16, C, rlist, rcount, k0, ks,
                        reinterpret_cast<RescoreLds<64> *>(keys)[wave]);
    return;
  }
  eval_wg<EB>(s, t, w, tab, layer, th, blockIdx.y, blockIdx.x, keys, pos, sh);
}

// The first controller round (nothing flagged, no value promoted yet) and the
// speculative mixed decode in one launch: workgroups [0, Hq n) evaluate the
// heads, the rest run two decode chunks each (threads [0, 512) and [512,
// 1024): the call's chunks in (sequence, KV head, chunk) order, a chunk past
// the last computed and not stored).  The decode reads only U, the scores
// and the block maxima, all final before this launch except a deferring
// step's ŝ′ outside U (resc != 0), which each decode wave computes for its
// own blocks before reading them; the evaluation reads no ŝ′.  So the
// heads' latency-bound chains of phases run beside the decode's streaming
// work.
template <int EB, int D, int CB>
__global__ __launch_bounds__(CTL_NT) void k_eval_decode(Shape s, Tier1 t, Step w, SeqTab tab, int layer,
                                                        Thresh th, const uint16_t *q16, float C, int resc) {
  extern __shared__ __align__(16) unsigned long long keys[];
  __shared__ uint16_t pos[MAX_NB];
  __shared__ CtlShared sh;
  const int nev = s.Hq * tab.n, x = blockIdx.x;
  if (x < nev) {
    eval_wg<EB>(s, t, w, tab, layer, th, x / s.Hq, x % s.Hq, keys, pos, sh);
    return;
  }
  static_assert(CTL_NT == 2 * 512, "two eight-wave decode chunks per workgroup");
  const int sub = threadIdx.x >> 9;
  int rem = 2 * (x - nev) + sub, i = 0;
  bool live = true;
  for (;; ++i) {
    if (i >= tab.n) {                   // past the last chunk: chunk 0 again, not stored
      live = false;
      i = 0;
      rem = 0;
      break;
    }
    const int cnt = s.Hkv * tab.nch[i];
    if (rem < cnt) break;
    rem -= cnt;
  }
  const int g = rem / tab.nch[i], ch = rem - g * tab.nch[i];
  typedef DecLds<D, CB, 4, false> DL;
  // a deferring step: each chunk's eight waves have a rescoring area each,
  // after the two chunks' decode areas
  RescoreLds<D> *rl = resc ? reinterpret_cast<RescoreLds<D> *>(reinterpret_cast<char *>(keys) + 2 * sizeof(DL)) + 8 * sub
                           : nullptr;
  decode_chunk<D, CB, 4, false>(s, t, w, tab, layer, i, g, ch, live, threadIdx.x & 511,
                                reinterpret_cast<DL *>(keys)[sub], q16, C, rl);
}

// Part 2, one workgroup per (sequence, KV head): rung 1 decisions; a group
// that widens plans its new key blocks, a group that stops takes its final
// decisions (rung 3 for heads above eps_key, rung 2, E_val, levels) and
// plans its value blocks.
__global__ __launch_bounds__(CTL_NT) void k_decide(Shape s, Tier1 t, Step w, SeqTab tab, int layer,
                                                   Thresh th, int round) {
  extern __shared__ unsigned long long keys[];
  __shared__ CtlShared sh;
  __shared__ int tmp[18];
  const int i = blockIdx.y, g = blockIdx.x;
  uint32_t *gs = w.gstat + (size_t)i * s.Hkv + g;
  // the group's state, and (lane hh of wave 0) head hh's state and E_val
  // ingredients from the evaluation (numerator with no value promoted,
  // denominator), read together
  const uint32_t gsv = *gs;
  const size_t oh = (size_t)i * s.Hq + g * s.G + threadIdx.x;
  uint32_t f = 0u;
  double ek = 0.0;
  int ss = 0;
  unsigned long long evn = 0ull, evd = 0ull;
  if (threadIdx.x < s.G) {
    f = w.hflags[oh];
    ek = w.ekey64[oh];
    ss = w.ssize[oh];
    evn = w.evs[2 * oh];
    evd = w.evs[2 * oh + 1];
  }
  if (gsv & 1u) {                             // group already final: nothing new to copy
    if (threadIdx.x == 0 && (gsv & 2u)) atomicOr(&w.plan[2], 2ull);
    return;
  }
  const int T = tab.T[i], NB = (T + BLOCK - 1) / BLOCK;
  const size_t unit = unit_of(s, tab.slot[i], layer, g);
  // rung-1 decisions of the group: lane hh of wave 0 takes head hh; "some
  // head widens" is the wave's ballot.  The E_val ingredients go to LDS so
  // that the head loop below indexes them freely.
  __shared__ uint32_t hf[4];
  __shared__ unsigned long long ssum[8];
  if (threadIdx.x < 64) {
    const int hh = threadIdx.x;
    const bool wid = hh < s.G && round < th.R1 && !(f & 4u) && ek > th.eps_key && ss < NB;
    const bool any = __ballot(wid) != 0ull;
    if (hh < s.G) {
      if (wid) {
        ss = min(NB, 2 * ss);
        f |= 2u;
      }
      // final round of this group: rung 3 for heads still above eps_key
      if (!any && !(f & 4u) && ek > th.eps_key) f |= 4u;
      hf[hh] = f;
      w.hflags[oh] = f;
      w.ssize[oh] = ss;
      ssum[2 * hh] = evn;
      ssum[2 * hh + 1] = evd;
    }
    if (hh == 0) sh.wid = any ? 1 : 0;
  }
  __syncthreads();
  if (sh.wid) {
    if (threadIdx.x == 0) atomicOr(&w.plan[2], 1ull);
    plan_group_keys(s, w, i, g, NB);
    return;
  }
  const uint8_t *V = w.V + ((size_t)i * s.Hkv + g) * s.NBmax;
  const float *eta = t.eta + unit * s.NBmax;
  unsigned long long sums[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) sums[k] = (k < 2 * s.G) ? ssum[k] : 0ull;
  int anyv = 0;
  if (th.fp16_values) {
    // FP16-values ablation: every block's values from tier 2, no rung 2
    uint8_t *Vw = w.V + ((size_t)i * s.Hkv + g) * s.NBmax;
    for (int b = threadIdx.x; b < NB; b += CTL_NT) Vw[b] = 1;
    anyv = 1;
  }
  for (int hh = 0; hh < s.G && !th.fp16_values; ++hh) {
    const int hq = g * s.G + hh;
    if (hf[hh] & 4u) continue;
    const unsigned long long nv = ssum[2 * hh], dv = ssum[2 * hh + 1];
    if ((double)nv / (double)dv > th.v_tol) {
      value_rung(s, t, w, th, i, g, hq, NB, unit, nv, dv, keys, sh);
      if (threadIdx.x == 0) hf[hh] |= 8u;
      anyv = 1;
    }
  }
  __syncthreads();
  if (anyv) {
    // E_val on the group's V: contributions of blocks without FP16 values
#pragma unroll
    for (int k = 0; k < 8; k += 2) sums[k] = 0ull;
    for (int b = threadIdx.x; b < NB; b += CTL_NT) {
      if (V[b]) continue;
      const double eb = (double)eta[b];
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        if (hh >= s.G) continue;
        const uint32_t Wt = w.Wt[((size_t)i * s.Hq + g * s.G + hh) * s.NBmax + b];
        sums[2 * hh] += (unsigned long long)ceil((double)(Wt + 65u) * W_UP * eb);
      }
    }
    unsigned long long dens[4];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) dens[hh] = sums[2 * hh + 1];
    block_sum_u64_8(sums, sh);
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) sums[2 * hh + 1] = dens[hh];
  }
  int any3 = 0;
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    if (hh >= s.G) continue;
    const size_t o = (size_t)i * s.Hq + g * s.G + hh;
    const uint32_t f = hf[hh];
    if (f & 4u) {
      any3 = 1;
      if (threadIdx.x == 0) {
        w.hlevel[o] = 3;
        w.eval64[o] = 0.0;
      }
    } else if (threadIdx.x == 0) {
      w.eval64[o] = (double)sums[2 * hh] / (double)sums[2 * hh + 1];
      w.hlevel[o] = (f & 8u) ? 2 : ((f & 2u) ? 1 : 0);
    }
  }
  // value promotions to copy: runs of V, extracted from an LDS copy
  if (anyv) {
    __shared__ uint8_t fv[MAX_NB];
    for (int b = threadIdx.x; b < NB; b += CTL_NT) fv[b] = V[b];
    __syncthreads();
    uint32_t *runs = w.runs + (((size_t)i * s.Hkv + g) * 2 + 1) * s.runmax;
    const int nrv = build_runs(fv, NB, runs, tmp);
    emit_runs(s, w, i * s.Hkv + g, 1, runs, nrv, tmp + 17);
  }
  if (threadIdx.x == 0) {
    *gs = 1u | (any3 ? 2u : 0u);
    if (any3) atomicOr(&w.plan[2], 2ull);
  }
  if (threadIdx.x < s.G) {
    // bit3 marks V_h non-empty; bits 8..15 the round the group stopped in
    w.hflags[(size_t)i * s.Hq + g * s.G + threadIdx.x] = (hf[threadIdx.x] & 0xffu) | ((uint32_t)round << 8);
  }
}

hipError_t launch_eval(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab, int layer,
                       const Thresh &th, int maxNB, const uint16_t *q, float C, const uint32_t *rlist,
                       int rcount, hipStream_t st) {
  const int n2 = max(64, pow2_at_least(maxNB));
  // rescoring workgroups: one wave per listed block, at most two per CU
  const int R = rcount > 0 ? std::min((rcount + CTL_NT / 64 - 1) / (CTL_NT / 64), 2 * std::max(s.ncu, 1)) : 0;
  const dim3 grid(s.Hq + R, tab.n), block(CTL_NT);
  const size_t rl = R ? (CTL_NT / 64) * (s.d == 128 ? sizeof(RescoreLds<128>) : sizeof(RescoreLds<64>)) : 0;
  const uint32_t lds = (uint32_t)std::max({sort_lds_bytes(n2), rl, EVAL_TOT_BYTES});
  switch ((maxNB + CTL_NT - 1) / CTL_NT) {   // blocks per thread
    case 1: return launch_k(k_eval<1>, grid, block, lds, st, s, t, w, tab, layer, th, q, C, rlist, rcount);
    case 2: return launch_k(k_eval<2>, grid, block, lds, st, s, t, w, tab, layer, th, q, C, rlist, rcount);
    case 3: return launch_k(k_eval<3>, grid, block, lds, st, s, t, w, tab, layer, th, q, C, rlist, rcount);
    default: return launch_k(k_eval<4>, grid, block, lds, st, s, t, w, tab, layer, th, q, C, rlist, rcount);
  }
}

// One workgroup of k_eval_decode fits a CU at a time (two thirds of the
// standalone decode's waves), so it pays while the call needs at most two
// rounds of workgroups: at 128K tokens, batch 1 (evaluation + decode 36.9 ->
// 24.7 us) and batch 2 (53.1 -> 48.4 us), not batch 4 (88.7 -> 94.1 us).
// The test hook's chunk shapes (8 or 16 blocks) keep separate launches.
bool eval_decode_fits(const Shape &s, const SeqTab &tab) {
  if (mix_chunk_blocks() != MIX_CB) return false;
  long long base = 0;
  for (int i = 0; i < tab.n; ++i) base += (long long)s.Hkv * ((tab.nbc[i + 1] - tab.nbc[i] + MIX_CB - 1) / MIX_CB);
  return (long long)s.Hq * tab.n + (base + 1) / 2 <= 2LL * std::max(s.ncu, 1);
}

hipError_t launch_eval_decode(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab0,
                              int layer, const Thresh &th, int maxNB, const uint16_t *q, float C,
                              bool resc, int *extra, hipStream_t st) {
  *extra = -1;
  if (!eval_decode_fits(s, tab0)) return hipSuccess;
  const int n2 = max(64, pow2_at_least(maxNB));
  const int nev = s.Hq * tab0.n;
  SeqTab tab = tab0;
  mix_chunk_counts(s, tab, MIX_CB, 2, nev);
  int total = 0, most = 0;
  for (int i = 0; i < tab.n; ++i) {
    const int NB = tab.nbc[i + 1] - tab.nbc[i];
    total += s.Hkv * tab.nch[i];
    most = std::max(most, (NB + tab.nch[i] - 1) / tab.nch[i]);
  }
  const dim3 grid(nev + (total + 1) / 2), block(CTL_NT);
  const bool c32 = most <= 32;
  size_t lds = sort_lds_bytes(n2);
  const size_t dl = s.d == 128 ? (c32 ? sizeof(DecLds<128, 32, 4, false>) : sizeof(DecLds<128, 48, 4, false>))
                               : (c32 ? sizeof(DecLds<64, 32, 4, false>) : sizeof(DecLds<64, 48, 4, false>));
  const size_t rl = resc ? 16 * (s.d == 128 ? sizeof(RescoreLds<128>) : sizeof(RescoreLds<64>)) : 0;
  lds = std::max({lds, 2 * dl + rl, EVAL_TOT_BYTES});
  const int eb = (maxNB + CTL_NT - 1) / CTL_NT;   // blocks per thread of the evaluation
  hipError_t e;
#define KVQ_ED(EB_, D_, CB_)                                                                        \
  e = launch_k(k_eval_decode<EB_, D_, CB_>, grid, block, (uint32_t)lds, st, s, t, w, tab, layer, th, q, C, \
               resc ? 1 : 0)
#define KVQ_ED_D(EB_)                          \
  if (s.d == 128) {                            \
    if (c32) KVQ_ED(EB_, 128, 32);             \
    else KVQ_ED(EB_, 128, 48);                 \
  } else {                                     \
    if (c32) KVQ_ED(EB_, 64, 32);              \
    else KVQ_ED(EB_, 64, 48);                  \
  }
  switch (eb) {
    case 1: KVQ_ED_D(1) break;
    case 2: KVQ_ED_D(2) break;
    case 3: KVQ_ED_D(3) break;
    default: KVQ_ED_D(4) break;
  }
#undef KVQ_ED_D
#undef KVQ_ED
  if (e == hipSuccess) *extra = nev;
  return e;
}

hipError_t launch_decide(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab,
                         int layer, const Thresh &th, int round, int maxNB, hipStream_t st) {
  const int n2 = max(64, pow2_at_least(maxNB));
  return launch_k(k_decide, dim3(s.Hkv, tab.n), dim3(CTL_NT), (uint32_t)sort_lds_bytes(n2), st, s,
                  t, w, tab, layer, th, round);
}

hipError_t launch_control(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab,
                          int layer, const Thresh &th, int round, int maxNB, hipStream_t st) {
  const hipError_t e = launch_eval(s, t, w, tab, layer, th, maxNB, nullptr, 0.0f, nullptr, 0, st);
  if (e != hipSuccess) return e;
  return launch_decide(s, t, w, tab, layer, th, round, maxNB, st);
}

// ---- rung 4 and the per-head outputs ---------------------------------------------

__global__ void k_finalize(Shape s, Step w, SeqTab tab, Thresh th, float *e_key, float *e_val,
                           int8_t *level) {
  const int i = blockIdx.x;
  __shared__ int n3;
  if (threadIdx.x == 0) n3 = 0;
  __syncthreads();
  for (int h = threadIdx.x; h < s.Hq; h += blockDim.x)
    if (w.hlevel[(size_t)i * s.Hq + h] == 3) atomicAdd(&n3, 1);
  __syncthreads();
  const bool all4 = th.force_dense ||
                    1000000ull * (unsigned long long)n3 > (unsigned long long)th.frac_ppm * s.Hq;
  for (int h = threadIdx.x; h < s.Hq; h += blockDim.x) {
    const size_t o = (size_t)i * s.Hq + h;
    const int lv = all4 ? 4 : w.hlevel[o];
    w.hlevel[o] = (int8_t)lv;
    level[o] = (int8_t)lv;
    e_key[o] = (lv >= 3) ? 0.0f : f32_up(w.ekey64[o]);
    e_val[o] = (lv >= 3) ? 0.0f : f32_up(w.eval64[o]);
  }
  __syncthreads();
  for (int g = threadIdx.x; g < s.Hkv; g += blockDim.x) {
    uint8_t dn = 0;
    for (int hh = 0; hh < s.G; ++hh) dn |= (w.hlevel[(size_t)i * s.Hq + g * s.G + hh] >= 3);
    w.gdense[(size_t)i * s.Hkv + g] = dn;
  }
}

hipError_t launch_finalize(const Shape &s, const Step &w, const SeqTab &tab, const Thresh &th,
                           float *e_key, float *e_val, int8_t *level, hipStream_t st) {
  return launch_k(k_finalize, dim3(tab.n), dim3(64), 0, st, s, w, tab, th, e_key, e_val, level);
}

}  // namespace kvq
