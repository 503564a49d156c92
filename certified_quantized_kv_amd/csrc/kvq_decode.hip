// kvq_decode.hip -- split-K decode attention over the mixed-precision cache
// and the dense FP16 fallback ("Runtime-Certified Bounded-Error Quantized
// Attention", Méthodologie §3: promoted blocks use FP16 keys, the tail stays
// INT8; rung 2 promotes values; rungs 3/4 recompute with full FP16 K and V,
// Méthodologie §1).
//
// Mixed mode, per (sequence, KV head, chunk of up to 48 blocks):
//   scores: FP16-key score on blocks of U_g, INT8 score elsewhere (both
//           already computed, log2 units);
//   values: FP16 from the staging buffer on blocks of V_g, INT4 dequantized
//           in registers as fmaf(scale, code, offset) elsewhere;
//   online softmax in fp32: the chunk's max M_h and sum l_h per head, and
//           o_h = sum_t 2^(x_t - M_h) v_t; the combine kernel merges chunks.
// Dense mode (groups with a head at level 3/4) is the kernel of
// kvq_dense.hip on the staged FP16 keys and values.
#include <algorithm>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_mixed.h"

namespace kvq {

// the chunk body (decode_chunk) and its LDS (DecLds): kvq_mixed.h
template <int D, int CB, int NP, bool FV>
__global__ __launch_bounds__(128 * NP) void k_decode_mixed(Shape s, Tier1 t, Step w, SeqTab tab, int layer) {
  __shared__ DecLds<D, CB, NP, FV> L;
  const int i = blockIdx.z, g = blockIdx.y, ch = blockIdx.x;
  if (ch >= tab.nch[i]) return;
  decode_chunk<D, CB, NP, FV>(s, t, w, tab, layer, i, g, ch, true, threadIdx.x, L);
}

// Blocks per chunk of the mixed decode: at most MIX_CB (48, eight waves), or
// 8 or 16 (four waves) while a test has selected them
// (kvq_selftest_launch_shape).  Outputs round differently with the chunking;
// no decision depends on it.
static int g_mix_cb = MIX_CB;
void set_mix_chunk_blocks(int cb) { g_mix_cb = (cb == 8 || cb == 16) ? cb : MIX_CB; }
int mix_chunk_blocks() { return g_mix_cb; }

// Chunks per sequence: at least ceil(NB / cb) (a chunk holds at most cb
// blocks), cut smaller until the call's workgroups are a multiple of the
// compute units, so that every unit gets the same number of equal chunks
// (with a few more workgroups than a multiple, some units run one chunk more
// than the others: measured 26.4 us against 22.4 us for 2049 against 2048
// blocks at batch 1 with 32-block chunks); at most one chunk per DEC_CB
// blocks (the partials buffer).  A pure function of the call, so the combine
// finds the same chunks.  With per_wg > 1 (k_eval_decode: two chunks per
// workgroup, one workgroup per CU, beside `extra` other workgroups) the
// workgroups of the launch, not the chunks, make the multiple.
void mix_chunk_counts(const Shape &s, SeqTab &tab, int cb, int per_wg, int extra) {
  const long long ncu = std::max(s.ncu, 1);
  long long total = 0;
  for (int i = 0; i < tab.n; ++i)
    total += (long long)s.Hkv * ((tab.nbc[i + 1] - tab.nbc[i] + cb - 1) / cb);
  const long long wgs = (total + per_wg - 1) / per_wg + extra;
  const long long want = per_wg * ((wgs + ncu - 1) / ncu * ncu - extra);
  for (int i = 0; i < tab.n; ++i) {
    const int NB = tab.nbc[i + 1] - tab.nbc[i];
    const long long base = (NB + cb - 1) / cb;
    const long long hi = std::max(1, (NB + DEC_CB - 1) / DEC_CB);
    long long n = total > 0 ? base * want / total : base;
    n = std::min(std::max(n, base), std::max(hi, base));
    tab.nch[i] = (int)n;
  }
}

template <bool FV>
static hipError_t launch_decode_fv(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab,
                                   dim3 grid, int cb, int most, int layer, hipStream_t st) {
  if (cb == 8) {
    if (s.d == 128)
      return launch_k(k_decode_mixed<128, 8, 2, FV>, grid, dim3(256), 0, st, s, t, w, tab, layer);
    return launch_k(k_decode_mixed<64, 8, 2, FV>, grid, dim3(256), 0, st, s, t, w, tab, layer);
  }
  if (cb == 16) {
    if (s.d == 128)
      return launch_k(k_decode_mixed<128, 16, 2, FV>, grid, dim3(256), 0, st, s, t, w, tab, layer);
    return launch_k(k_decode_mixed<64, 16, 2, FV>, grid, dim3(256), 0, st, s, t, w, tab, layer);
  }
  // eight waves; the 32-block build when every chunk fits it (its fully
  // unrolled block loop is shorter: 22.2 against 24.2 us at batch 1, 128K)
  static_assert(MIX_CB == 48, "the default chunk is the eight-wave kernel");
  if (most <= 32) {
    if (s.d == 128)
      return launch_k(k_decode_mixed<128, 32, 4, FV>, grid, dim3(512), 0, st, s, t, w, tab, layer);
    return launch_k(k_decode_mixed<64, 32, 4, FV>, grid, dim3(512), 0, st, s, t, w, tab, layer);
  }
  if (s.d == 128)
    return launch_k(k_decode_mixed<128, 48, 4, FV>, grid, dim3(512), 0, st, s, t, w, tab, layer);
  return launch_k(k_decode_mixed<64, 48, 4, FV>, grid, dim3(512), 0, st, s, t, w, tab, layer);
}

hipError_t launch_decode(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab0,
                         int layer, bool values, hipStream_t st) {
  const int cb = g_mix_cb;
  SeqTab tab = tab0;
  mix_chunk_counts(s, tab, cb, 1, 0);
  int xmax = 1, most = 0;
  for (int i = 0; i < tab.n; ++i) {
    const int NB = tab.nbc[i + 1] - tab.nbc[i];
    xmax = std::max(xmax, tab.nch[i]);
    most = std::max(most, (NB + tab.nch[i] - 1) / tab.nch[i]);
  }
  const dim3 grid(xmax, s.Hkv, tab.n);
  return values ? launch_decode_fv<true>(s, t, w, tab, grid, cb, most, layer, st)
                : launch_decode_fv<false>(s, t, w, tab, grid, cb, most, layer, st);
}

// Merges the chunk partials of each (sequence, query head): mode 0 reads the
// dense partials for heads at level 3/4 and the mixed ones for the others,
// mode 1 the mixed ones and mode 2 the dense ones for every head.  One workgroup per
// (query head, sequence, quarter of the channels): the chunk maxima and
// weights first (every quarter computes them), then 256 / (d/4) groups of
// channel-threads each sum a share of the chunks with four independent
// accumulators; the shares are added in LDS.
constexpr int COMB_MAXCH = 1024;
static_assert((MAX_NB + DEC_CB - 1) / DEC_CB <= COMB_MAXCH, "chunk weights fit in LDS");

// With `level` non-null (a certified step in which no head reached rung 3, so
// no rung 4 either) the workgroup of channel quarter 0 also writes the
// head's outputs: level, and E_key, E_val rounded up to binary32 (mode 3:
// from the first round's evaluation sums, the group decisions not having run).
__global__ __launch_bounds__(256) void k_combine(Shape s, Step w, SeqTab tab, float *out, int mode,
                                                 float *e_key, float *e_val, int8_t *level,
                                                 int mix_cb) {
  __shared__ float fw[COMB_MAXCH];
  __shared__ float red[256];
  __shared__ float wred[4];
  const int i = blockIdx.y, hq = blockIdx.x, cq = blockIdx.z;
  const int D = s.d, G = s.G, g = hq / G, h = hq % G, CQ = D / 4;
  if (level && cq == 0 && threadIdx.x == 0) {
    const size_t o = (size_t)i * s.Hq + hq;
    if (mode == 3) {
      // first round, no head flagged: consistent, E_key <= eps_key, no value
      // promoted (E_val <= v_tol), nothing widened -> level 0
      const double ev = (double)w.evs[2 * o] / (double)w.evs[2 * o + 1];
      w.eval64[o] = ev;
      w.hlevel[o] = 0;
      level[o] = 0;
      e_key[o] = f32_up(w.ekey64[o]);
      e_val[o] = f32_up(ev);
    } else {
      level[o] = w.hlevel[o];
      e_key[o] = f32_up(w.ekey64[o]);
      e_val[o] = f32_up(w.eval64[o]);
    }
  }
  const bool dense = mode == 2 || (mode == 0 && w.hlevel[(size_t)i * s.Hq + hq] >= 3);
  const int cb = dense ? DEC_CB : mix_cb;
  const int NB = (tab.T[i] + BLOCK - 1) / BLOCK, nch = dense ? (NB + cb - 1) / cb : tab.nch[i];
  const float *part = (dense ? w.partd : w.part) + (((size_t)i * s.Hkv + g) * s.nchmax * G + h) * (D + 2);
  const size_t stride = (size_t)G * (D + 2);
  const int parts = 256 / CQ, c = cq * CQ + threadIdx.x % CQ, pp = threadIdx.x / CQ;
  // every load of the workgroup goes out at once: the chunk maxima and sums
  // of this thread's chunks t + 256 j, and the first PF partial outputs of its
  // channel (chunks pp + parts j); the rest of the partials stream later
  constexpr int MJ = COMB_MAXCH / 256, PF = 16;
  float mk[MJ], lk[MJ], pv[PF];
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    const int k = threadIdx.x + 256 * j;
    mk[j] = k < nch ? part[k * stride + D] : -INFINITY;
    lk[j] = k < nch ? part[k * stride + D + 1] : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    const int k = pp + parts * j;
    pv[j] = k < nch ? part[k * stride + c] : 0.0f;
  }
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < MJ; ++j) m = fmaxf(m, mk[j]);
  m = bfly_max<64>(m);
  if ((threadIdx.x & 63) == 0) wred[threadIdx.x >> 6] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
  __syncthreads();
  float l = 0.0f;
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    const int k = threadIdx.x + 256 * j;
    if (k < nch) {
      const float f = exp2f(mk[j] - M);
      fw[k] = f;
      l = fmaf(lk[j], f, l);
    }
  }
  l = bfly_sum<64>(l);
  if ((threadIdx.x & 63) == 0) wred[threadIdx.x >> 6] = l;
  __syncthreads();
  const float L = wred[0] + wred[1] + wred[2] + wred[3];
  // accumulators: chunk j of this thread goes to a[j % 4] when its group of
  // four chunks is complete, to a[0] otherwise (the tail), in increasing j
  float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    const int k = pp + parts * j;
    if (k < nch) {
      const bool full = pp + parts * ((j & ~3) + 3) < nch;
      const float f = fw[k];
      if (full) a[j & 3] = fmaf(pv[j], f, a[j & 3]);
      else a[0] = fmaf(pv[j], f, a[0]);
    }
  }
  int k = pp + parts * PF;
  for (; k + 3 * parts < nch; k += 4 * parts) {
    a[0] = fmaf(part[k * stride + c], fw[k], a[0]);
    a[1] = fmaf(part[(k + parts) * stride + c], fw[k + parts], a[1]);
    a[2] = fmaf(part[(k + 2 * parts) * stride + c], fw[k + 2 * parts], a[2]);
    a[3] = fmaf(part[(k + 3 * parts) * stride + c], fw[k + 3 * parts], a[3]);
  }
  for (; k < nch; k += parts) a[0] = fmaf(part[k * stride + c], fw[k], a[0]);
  const float a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
  red[threadIdx.x] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  if (threadIdx.x < CQ) {
    float sum = 0.0f;
    for (int q = 0; q < parts; ++q) sum += red[q * CQ + threadIdx.x];
    out[((size_t)i * s.Hq + hq) * D + c] = sum / L;
  }
}

hipError_t launch_combine(const Shape &s, const Step &w, const SeqTab &tab0, float *out, int mode,
                          float *e_key, float *e_val, int8_t *level, int fused_extra, hipStream_t st) {
  SeqTab tab = tab0;
  if (mode != 2) {
    if (fused_extra >= 0)
      mix_chunk_counts(s, tab, g_mix_cb, 2, fused_extra);
    else
      mix_chunk_counts(s, tab, g_mix_cb, 1, 0);
  }
  return launch_k(k_combine, dim3(s.Hq, tab.n, 4), dim3(256), 0, st, s, w, tab, out, mode, e_key,
                  e_val, level, g_mix_cb);
}

}  // namespace kvq
