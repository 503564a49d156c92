// kvq_dense.hip -- standard dense decode attention over an FP16 KV cache held
// in device memory: the reference point against which the pages state the
// cost of certification ("Runtime-Certified Bounded-Error Quantized
// Attention", Résultats: slowdown versus dense attention at 8K-128K).
//
// Per (sequence, KV head, chunk of DEC_CB = 8 blocks) one workgroup; wave w takes
// blocks b0 + w, b0 + w + 4, ... of the chunk, 32 tokens at a time:
//   scores  s_ht = q_h . k_t on the matrix cores: v_mfma_f32_16x16x32_f16
//           with rows = the group's query heads (zero rows above G),
//           k = 32 channels, n = 16 tokens; exact fp16 products summed in
//           fp32 (log2 units after the 1/sqrt(d) log2(e) scale);
//   softmax online per head in fp32 (running max m_h, sum l_h);
//   P.V     on the vector units: lane (token group j, channel slice c)
//           accumulates p_ht v_tc for its slice with fp32 fma of fp16 values.
// The four waves' partials are merged in LDS into one (m, l, o[d]) per head
// and chunk; the combine kernel merges the chunks.  K and V are read once
// (non-temporal loads).
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

// One chunk (DEC_CB blocks) of sequence i, KV head g: q of the group's
// heads at qg ([G][D] fp16), K and V rows of the sequence at Kb / Vb with
// rowstride halves between tokens; partials to w.partd.
template <int D>
__device__ __forceinline__ void dense_chunk(const Shape &s, const Step &w, int i, int g, int ch,
                                            int T, const uint16_t *qg, const uint16_t *Kb,
                                            const uint16_t *Vb, size_t rowstride) {
  constexpr int KS = D / 32;                 // MFMA k-steps over the channels
  constexpr int CPL = D / 16;                // channels per lane in P.V
  constexpr int STEP = 32;                   // tokens per step (two 16-token tiles)
  const int NB = (T + BLOCK - 1) / BLOCK;
  const int b0 = ch * DEC_CB;
  if (b0 >= NB) return;
  const int b1 = min(NB, b0 + DEC_CB);
  const int G = s.G;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const float C = (float)(1.4426950408889634 / sqrt((double)D));

  __shared__ __align__(16) float ps[4][STEP][4];        // p per wave: [token][head]
  __shared__ float sm[4][4], sl[4][4];
  __shared__ float so[4][4][D];

  // A operand: row r = lane & 15 (query head r of the group, zero above G),
  // k = channels 32 ks + 8 (lane >> 4) + 0..7
  h8v qa[KS];
  {
    const int r = lane & 15;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      h8v x = (h8v){0, 0, 0, 0, 0, 0, 0, 0};
      if (r < G) {
        const uint16_t *qp = qg + (size_t)r * D + 32 * ks + 8 * (lane >> 4);
        x = *(const h8v *)qp;
      }
      qa[ks] = x;
    }
  }

  float m[4], l[4], o[4][CPL];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[h][c] = 0.0f;
  }
  const int tj = lane >> 4;                  // P.V: token j = tj + 4 r, r = 0..7
  const int c0 = CPL * (lane & 15);          // P.V: channel slice

  for (int b = b0 + wave; b < b1; b += 4) {
    for (int t0 = b * BLOCK; t0 < min(T, (b + 1) * BLOCK); t0 += STEP) {
      // ---- loads of the step: K as the MFMA B operand, V slices -------------
      h8v kb[2][KS];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int tok = min(t0 + tt * 16 + (lane & 15), T - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kb[tt][ks] = __builtin_nontemporal_load(
              (const h8v *)(Kb + (size_t)tok * rowstride + 32 * ks + 8 * (lane >> 4)));
      }
      typedef _Float16 hc __attribute__((ext_vector_type(CPL)));
      hc vv[STEP / 4];
#pragma unroll
      for (int r = 0; r < STEP / 4; ++r) {
        const int tok = min(t0 + tj + 4 * r, T - 1);
        vv[r] = __builtin_nontemporal_load((const hc *)(Vb + (size_t)tok * rowstride + c0));
      }
      // ---- scores --------------------------------------------------------------
      float x[2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f4v acc = (f4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[ks], kb[tt][ks], acc, 0, 0, 0);
        const bool ok = lane < 16 && t0 + tt * 16 + lane < T;
#pragma unroll
        for (int h = 0; h < 4; ++h) x[tt][h] = (ok && h < G) ? acc[h] * C : -INFINITY;
      }
      // ---- online softmax (lanes 0..15 hold the scores) -------------------------
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        float mx = bfly_max<16>(fmaxf(x[0][h], x[1][h]));
        mx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 0));
        const float mn = fmaxf(m[h], mx);
        const float sc = (mn == -INFINITY) ? 1.0f : exp2f(m[h] - mn);
        m[h] = mn;
        l[h] *= sc;
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[h][c] *= sc;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const float p = (x[tt][h] == -INFINITY) ? 0.0f : exp2f(x[tt][h] - mn);
          if (lane < 16) ps[wave][tt * 16 + lane][h] = p;
          l[h] += p;
        }
      }
      wave_lds_sync();
      // ---- P.V -------------------------------------------------------------------
#pragma unroll
      for (int r = 0; r < STEP / 4; ++r) {
        const int j = tj + 4 * r;
        const f4v p = *(const f4v *)&ps[wave][j][0];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float vf = (float)vv[r][c];
#pragma unroll
          for (int h = 0; h < 4; ++h) o[h][c] = fmaf(p[h], vf, o[h][c]);
        }
      }
      wave_lds_sync();
    }
  }
  // ---- wave partials: o over the four token groups, l over lanes 0..15 ---------
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    l[h] = bfly_sum<64>(l[h]);               // lanes >= 16 added zeros
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float v = o[h][c];
      v += xor_lane_f<16>(v);
      v += xor_lane_f<32>(v);
      o[h][c] = v;
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int c = 0; c < CPL; ++c) so[wave][h][c0 + c] = o[h][c];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      sm[wave][h] = m[h];
      sl[wave][h] = l[h];
    }
  }
  __syncthreads();
  // ---- merge the four waves: thread = (head, channel) ----------------------------
  const size_t ig = (size_t)i * s.Hkv + g;
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int h = idx / D, c = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) M = fmaxf(M, sm[q][h]);
    float acc = 0.0f, L = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (sm[q][h] == -INFINITY) continue;
      const float f = exp2f(sm[q][h] - M);
      acc = fmaf(so[q][h][c], f, acc);
      L = fmaf(sl[q][h], f, L);
    }
    float *part = w.partd + ((ig * s.nchmax + ch) * G + h) * (size_t)(D + 2);
    part[c] = acc;
    if (c == 0) {
      part[D] = M;
      part[D + 1] = L;
    }
  }
}

// Comparator: FP16 K and V resident in device memory, [n][tcap][Hkv][d].
template <int D>
__global__ __launch_bounds__(256) void k_dense_vram(Shape s, Step w, DenseArgs a) {
  const int i = blockIdx.z, g = blockIdx.y;
  dense_chunk<D>(s, w, i, g, blockIdx.x, a.T[i], a.q + ((size_t)i * s.Hq + g * s.G) * D,
                 a.k + ((size_t)i * a.tcap * s.Hkv + g) * D,
                 a.v + ((size_t)i * a.tcap * s.Hkv + g) * D, (size_t)s.Hkv * D);
}

// Rungs 3 and 4: the groups marked dense, from their staged FP16 K and V.
template <int D>
__global__ __launch_bounds__(256) void k_dense_staged(Shape s, Step w, SeqTab tab, int layer,
                                                      const uint16_t *q16) {
  const int i = blockIdx.z, g = blockIdx.y;
  const size_t ig = (size_t)i * s.Hkv + g;
  if (!w.gdense[ig]) return;
  dense_chunk<D>(s, w, i, g, blockIdx.x, tab.T[i], q16 + ((size_t)i * s.Hq + g * s.G) * D,
                 w.stage_k + stage_k_area(s, i, g, tab.slot[i], layer) * s.Tmax * D,
                 w.stage_v + ig * s.Tmax * D, (size_t)D);
}

hipError_t launch_dense_staged(const Shape &s, const Step &w, const SeqTab &tab, int layer,
                               const uint16_t *q16, int maxNB, hipStream_t st) {
  dim3 grid((maxNB + DEC_CB - 1) / DEC_CB, s.Hkv, tab.n);
  if (s.d == 128)
    return launch_k(k_dense_staged<128>, grid, dim3(256), 0, st, s, w, tab, layer, q16);
  return launch_k(k_dense_staged<64>, grid, dim3(256), 0, st, s, w, tab, layer, q16);
}

hipError_t launch_dense_vram(const Shape &s, const Step &w, const DenseArgs &a, int maxNB,
                             hipStream_t st) {
  dim3 grid((maxNB + DEC_CB - 1) / DEC_CB, s.Hkv, a.n);
  if (s.d == 128) return launch_k(k_dense_vram<128>, grid, dim3(256), 0, st, s, w, a);
  return launch_k(k_dense_vram<64>, grid, dim3(256), 0, st, s, w, a);
}

}  // namespace kvq
