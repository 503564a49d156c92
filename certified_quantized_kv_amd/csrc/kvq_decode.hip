// kvq_decode.hip -- split-K decode attention over the mixed-precision cache
// and the dense FP16 fallback ("Runtime-Certified Bounded-Error Quantized
// Attention", Méthodologie §3: promoted blocks use FP16 keys, the tail stays
// INT8; rung 2 promotes values; rungs 3/4 recompute with full FP16 K and V,
// Méthodologie §1).
//
// Mixed mode, per (sequence, KV head, chunk of 16 blocks):
//   scores: FP16-key score on blocks of U_g, INT8 score elsewhere (both
//           already computed, log2 units);
//   values: FP16 from the staging buffer on blocks of V_g, INT4 dequantized
//           in registers as fmaf(scale, code, offset) elsewhere;
//   online softmax in fp32: the chunk's max M_h and sum l_h per head, and
//           o_h = sum_t 2^(x_t - M_h) v_t; the combine kernel merges chunks.
// Dense mode (groups with a head at level 3/4): scores are the canonical
// FP16-key chains recomputed from the staged keys, values FP16 throughout.
// The four query heads of a KV head share each value load.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

template <int D, bool DENSE>
__global__ __launch_bounds__(256) void k_decode(Shape s, Tier1 t, Step w, SeqTab tab, int layer) {
  constexpr int CT = DEC_CB * BLOCK;              // tokens per chunk
  constexpr int CPL = D / 64;                     // channels per lane
  const int i = blockIdx.z, g = blockIdx.y, ch = blockIdx.x;
  const int T = tab.T[i], NB = (T + BLOCK - 1) / BLOCK;
  const int b0 = ch * DEC_CB;
  if (b0 >= NB) return;
  const size_t ig = (size_t)i * s.Hkv + g;
  if (DENSE && !w.gdense[ig]) return;
  const int G = s.G;
  const int t0 = b0 * BLOCK, nt = min(T, (b0 + DEC_CB) * BLOCK) - t0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t u = unit_of(s, tab.slot[i], layer, g);
  const uint8_t *U = w.U + ig * s.NBmax;
  const uint8_t *V = w.V + ig * s.NBmax;

  __shared__ float ps[4][CT];
  __shared__ float red[4][4][D];
  __shared__ float sM[4], sL[4];

  // ---- scores ------------------------------------------------------------------
  for (int idx = threadIdx.x; idx < G * nt; idx += 256) {
    const int h = idx / nt, tt = idx % nt;
    const int tok = t0 + tt;
    const int hq = g * G + h;
    float x;
    if (DENSE) {
      const uint16_t *row = w.stage_k + (ig * s.Tmax + tok) * D;
      const float *q = w.qp + ((size_t)i * s.Hq + hq) * D;
      float acc = 0.0f;
      for (int c = 0; c < D; ++c) acc = fmaf(q[c], h2f(row[c]), acc);
      x = acc;
    } else {
      const size_t o = ((size_t)i * s.Hq + hq) * s.Tmax + tok;
      x = U[tok / BLOCK] ? w.sp[o] : w.shat[o];
    }
    ps[h][tt] = x;
  }
  __syncthreads();
  if (wave < G) {
    float m = -INFINITY;
    for (int tt = lane; tt < nt; tt += 64) m = fmaxf(m, ps[wave][tt]);
    m = bfly_max<64>(m);
    float l = 0.0f;
    for (int tt = lane; tt < nt; tt += 64) {
      const float p = exp2f(ps[wave][tt] - m);
      ps[wave][tt] = p;
      l += p;
    }
    l = bfly_sum<64>(l);
    if (lane == 0) {
      sM[wave] = m;
      sL[wave] = l;
    }
  }
  __syncthreads();

  // ---- P.V ---------------------------------------------------------------------
  float o[4][CPL];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int k = 0; k < CPL; ++k) o[h][k] = 0.0f;
  const int per = (nt + 3) / 4;
  const int ta = wave * per, tb = min(nt, ta + per);
  const uint16_t *sv = w.stage_v + ig * s.Tmax * D;
  for (int tt = ta; tt < tb; ++tt) {
    const int tok = t0 + tt;
    float v[CPL];
    if (DENSE || V[tok / BLOCK]) {
      if (CPL == 2) {
        const uint32_t pr = *(const uint32_t *)(sv + (size_t)tok * D + 2 * lane);
        v[0] = h2f((uint16_t)(pr & 0xffffu));
        v[CPL - 1] = h2f((uint16_t)(pr >> 16));
      } else {
        v[0] = h2f(sv[(size_t)tok * D + lane]);
      }
    } else {
      const size_t row = u * s.Tmax + tok;
      const int c0 = CPL * lane;
      const uint32_t meta = t.vmeta[row * (D / VGROUP) + c0 / VGROUP];
      const float sc = h2f((uint16_t)(meta & 0xffffu)), of = h2f((uint16_t)(meta >> 16));
      const uint8_t byte = t.vcodes[row * (D / 2) + c0 / 2];
      if (CPL == 2) {
        v[0] = fmaf(sc, (float)(byte & 15), of);
        v[CPL - 1] = fmaf(sc, (float)(byte >> 4), of);
      } else {
        v[0] = fmaf(sc, (float)((lane & 1) ? (byte >> 4) : (byte & 15)), of);
      }
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      if (h < G) {
        const float p = ps[h][tt];
#pragma unroll
        for (int k = 0; k < CPL; ++k) o[h][k] = fmaf(p, v[k], o[h][k]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int k = 0; k < CPL; ++k) red[wave][h][CPL * lane + k] = o[h][k];
  __syncthreads();
  float *part = (DENSE ? w.partd : w.part) + ((ig * s.nchmax + ch) * G) * (size_t)(D + 2);
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int h = idx / D, c = idx % D;
    part[(size_t)h * (D + 2) + c] = red[0][h][c] + red[1][h][c] + red[2][h][c] + red[3][h][c];
  }
  if (threadIdx.x < G) {
    part[(size_t)threadIdx.x * (D + 2) + D] = sM[threadIdx.x];
    part[(size_t)threadIdx.x * (D + 2) + D + 1] = sL[threadIdx.x];
  }
}

hipError_t launch_decode(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab,
                         int layer, int maxNB, bool dense, hipStream_t st) {
  dim3 grid((maxNB + DEC_CB - 1) / DEC_CB, s.Hkv, tab.n);
  if (s.d == 128) {
    if (dense)
      hipLaunchKernelGGL((k_decode<128, true>), grid, dim3(256), 0, st, s, t, w, tab, layer);
    else
      hipLaunchKernelGGL((k_decode<128, false>), grid, dim3(256), 0, st, s, t, w, tab, layer);
  } else {
    if (dense)
      hipLaunchKernelGGL((k_decode<64, true>), grid, dim3(256), 0, st, s, t, w, tab, layer);
    else
      hipLaunchKernelGGL((k_decode<64, false>), grid, dim3(256), 0, st, s, t, w, tab, layer);
  }
  return hipGetLastError();
}

// Merges the chunk partials of each (sequence, query head): levels 3/4 read
// the dense partials, the others the mixed ones.
__global__ void k_combine(Shape s, Step w, SeqTab tab, float *out) {
  const int i = blockIdx.y, hq = blockIdx.x, c = threadIdx.x;
  const int D = s.d, G = s.G, g = hq / G, h = hq % G;
  const int NB = (tab.T[i] + BLOCK - 1) / BLOCK, nch = (NB + DEC_CB - 1) / DEC_CB;
  const bool dense = w.hlevel[(size_t)i * s.Hq + hq] >= 3;
  const float *part = (dense ? w.partd : w.part) + (((size_t)i * s.Hkv + g) * s.nchmax * G + h) * (D + 2);
  const size_t stride = (size_t)G * (D + 2);
  float M = -INFINITY;
  for (int k = 0; k < nch; ++k) M = fmaxf(M, part[k * stride + D]);
  float l = 0.0f, acc = 0.0f;
  for (int k = 0; k < nch; ++k) {
    const float f = exp2f(part[k * stride + D] - M);
    l = fmaf(part[k * stride + D + 1], f, l);
    if (c < D) acc = fmaf(part[k * stride + c], f, acc);
  }
  if (c < D) out[((size_t)i * s.Hq + hq) * D + c] = acc / l;
}

hipError_t launch_combine(const Shape &s, const Step &w, const SeqTab &tab, float *out,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_combine, dim3(s.Hq, tab.n), dim3(s.d), 0, st, s, w, tab, out);
  return hipGetLastError();
}

}  // namespace kvq
