// kvq_rescore.h -- INT8 scores ŝ′ of single blocks, for a step whose
// scoring pass stored none ("Runtime-Certified Bounded-Error Quantized
// Attention", Méthodologie §3: the INT8 pass; the decode reads ŝ′ only on
// blocks outside the promoted union U).
//
// One wave per block (sequence i, KV head g, block b), the same arithmetic as
// the pass in kvq_score.hip: q′ and the limbs of A per head, the exact
// integer core on the matrix cores, D_t rounded once from fp64, β as the fma
// chain over the channels in ascending order; ŝ′ of the block's 64 tokens
// stored.  A block's loads all go out before their first use.  Run over a
// list of blocks by k_rescore_int8 (kvq_score.hip) and the evaluation's
// extra workgroups (kvq_control.hip), and by the fused first round's decode
// chunks for their own blocks outside U (kvq_mixed.h).
#pragma once
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

typedef int rs_v4i __attribute__((ext_vector_type(4)));

// LDS of one wave
template <int D>
struct alignas(16) RescoreLds {
  int8_t As[16][D + 16];   // A limbs (row 4 h + l), rows padded (bank spread)
  float Qs[4][D];          // q′ rows (head slots)
  float Us[D];             // off + 128 s per channel
  float Bs[4];             // β per head slot
};

// Block b of (sequence i, KV head g) by the calling wave.  NTS: the scores
// go out as non-temporal stores and every load of the block goes out at once
// (a list whose scores a later launch reads); without it (a decode wave
// rescoring its own blocks, its stage registers live), the key codes load
// one 64-channel slice at a time, and the scores are plain stores that the
// same wave's later loads of those addresses observe (the wave's memory
// operations reach the caches in program order).
template <int D, bool NTS>
__device__ inline void rescore_block(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab,
                                     int layer, const uint16_t *__restrict__ q16, float C, int i, int g,
                                     int b, RescoreLds<D> &L) {
  constexpr int CW = D / 16;
  constexpr int NKS = D / 64;
  constexpr int AST = D + 16;
  typedef rs_v4i v4i;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 4, jc = lane & 15;
  const int G = s.G;
  const int hs = h < G ? h : 0;
  const size_t uu = unit_of(s, tab.slot[i], layer, g);
  // the loads of the block: codes, metadata, q slice
  constexpr int NKB = NTS ? NKS : 1;            // code slices held at once
  v4i Bn[NKB][4];
  const uint8_t *kc = t.kcodes + (uu * s.NBmax + b) * (size_t)(BLOCK * D);
  auto load_codes = [&](int ks, v4i *dst) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      dst[nt] = __builtin_nontemporal_load((const v4i *)(kc + ((size_t)((ks * 4 + nt) * 64 + lane)) * 16));
  };
  if (NTS) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) load_codes(ks, Bn[ks % NKB]);
  }
  uint32_t kb[CW];
  const uint32_t *km = t.kmeta + (uu * s.NBmax + b) * D + jc * CW;
#pragma unroll
  for (int c = 0; c < CW; ++c) kb[c] = km[c];
  uint32_t qb[CW / 2];
  const uint32_t *qs = (const uint32_t *)(q16 + ((size_t)i * s.Hq + g * G + hs) * D + jc * CW);
#pragma unroll
  for (int c = 0; c < CW / 2; ++c) qb[c] = qs[c];
  // q′, a = q′ s, the exponent and the limbs (lane (h, jc): head slot h,
  // channels jc CW ..); q′ rows and off + 128 s into LDS for the chains
  float qv[CW], a[CW];
  float am = 0.0f;
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    qv[c] = h2f((uint16_t)(qb[c / 2] >> (16 * (c % 2)))) * C;
    const float sv = h2f((uint16_t)(kb[c] & 0xffffu));
    a[c] = qv[c] * sv;
    am = fmaxf(am, fabsf(a[c]));
    L.Qs[h][jc * CW + c] = qv[c];
    if (h == 0) L.Us[jc * CW + c] = fmaf(128.0f, sv, h2f((uint16_t)(kb[c] >> 16)));
  }
  am = bfly_max<16>(am);
  const bool zero = !(am > 0.0f);
  const int e = zero ? 0 : ilogb_f(am) - 21;
  uint32_t l0w[CW / 4], l1w[CW / 4], l2w[CW / 4];
#pragma unroll
  for (int c = 0; c < CW / 4; ++c) l0w[c] = l1w[c] = l2w[c] = 0u;
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    const int A = (int)rintf(ldexpf(a[c], -e));
    const int L0 = ((A + 128) & 255) - 128;
    const int A1 = (A - L0) >> 8;
    const int L1 = ((A1 + 128) & 255) - 128;
    const int L2 = (A1 - L1) >> 8;
    l0w[c / 4] |= ((uint32_t)L0 & 255u) << (8 * (c % 4));
    l1w[c / 4] |= ((uint32_t)L1 & 255u) << (8 * (c % 4));
    l2w[c / 4] |= ((uint32_t)L2 & 255u) << (8 * (c % 4));
  }
  {
    int8_t *row = &L.As[h * 4][jc * CW];
#pragma unroll
    for (int c = 0; c < CW / 4; ++c) {
      ((uint32_t *)(row + 0 * AST))[c] = l0w[c];
      ((uint32_t *)(row + 1 * AST))[c] = l1w[c];
      ((uint32_t *)(row + 2 * AST))[c] = l2w[c];
      ((uint32_t *)(row + 3 * AST))[c] = 0u;
    }
  }
  wave_lds_sync();
  if (lane < 4) {                               // β of head slot lane
    // 16-byte LDS reads, eight of each operand in flight ahead of the
    // chain's fmas (which stay in ascending channel order)
    float beta = 0.0f;
#pragma unroll
    for (int c0 = 0; c0 < D; c0 += 32) {
      float4 q4[8], u4[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        q4[x] = *(const float4 *)&L.Qs[lane][c0 + 4 * x];
        u4[x] = *(const float4 *)&L.Us[c0 + 4 * x];
      }
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        beta = fmaf(q4[x].x, u4[x].x, beta);
        beta = fmaf(q4[x].y, u4[x].y, beta);
        beta = fmaf(q4[x].z, u4[x].z, beta);
        beta = fmaf(q4[x].w, u4[x].w, beta);
      }
    }
    L.Bs[lane] = beta;
  }
  v4i acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = (v4i){0, 0, 0, 0};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (!NTS) load_codes(ks, Bn[0]);
    const v4i Aop = *(const v4i *)&L.As[lane & 15][ks * 64 + 16 * (lane >> 4)];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      acc[nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aop, Bn[ks % NKB][nt], acc[nt], 0, 0, 0);
  }
  wave_lds_sync();
  const float pb = L.Bs[h];
  const float sc = ldexpf(1.0f, e);
  float *dst = w.shat + ((size_t)i * s.Hq + g * G + hs) * s.Tmax + (size_t)b * BLOCK;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const double Dd = fma((double)acc[nt][2], 65536.0, fma((double)acc[nt][1], 256.0, (double)acc[nt][0]));
    const float v = fmaf((float)Dd, sc, pb);
    if (NTS) __builtin_nontemporal_store(v, &dst[nt * 16 + jc]);
    else dst[nt * 16 + jc] = v;
  }
  wave_lds_sync();
}

// Units k0, k0 + kstride, ... of list[0 .. count) (entry ig << 16 | b,
// ig = i Hkv + g) by the calling wave.
template <int D>
__device__ inline void rescore_units(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab,
                                     int layer, const uint16_t *__restrict__ q16, float C,
                                     const uint32_t *__restrict__ list, int count, int k0, int kstride,
                                     RescoreLds<D> &L) {
  for (int k = k0; k < count; k += kstride) {
    const uint32_t ent = list[k];
    const int ig = (int)(ent >> 16), b = (int)(ent & 0xffffu);
    const int i = ig / s.Hkv, g = ig - i * s.Hkv;
    rescore_block<D, true>(s, t, w, tab, layer, q16, C, i, g, b, L);
  }
}

}  // namespace kvq
