// kvq_mixed.h -- one split-K chunk of the mixed-precision decode
// ("Runtime-Certified Bounded-Error Quantized Attention", Méthodologie §3:
// promoted blocks use FP16 keys, the tail stays INT8; rung 2 promotes
// values).  Run by k_decode_mixed (one chunk per workgroup) and by the first
// controller round's launch, k_eval_decode (two chunks per workgroup beside
// the heads' evaluation).
#pragma once
#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_rescore.h"

namespace kvq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Mixed decode.  Per block, sum_t p_ht v_tc with v = off_tj + s_tj code_tc
// splits into sum_t p_ht off_tj (VALU, per group) and the contraction
// sum_t (p_ht s_tj) code_tc on the matrix cores: A = fixed-point p*s as three
// signed byte limbs (rows: head x limb, k: 64 tokens), B = the INT4 codes
// (k: tokens, n: 16 channels), one v_mfma_i32_16x16x64_i8 per 16 channels.
//
// Per (sequence, KV head, chunk of CB blocks) one workgroup of 2 NP waves;
// wave w takes half w % 2 of the channels of blocks b0 + w / 2,
// b0 + w / 2 + NP, ..., so a block's scores and exponentials are read and
// formed by two waves.  The
// chunk's softmax reference M_h is the largest block maximum of the scores in
// use (FP16 on blocks of U, INT8 elsewhere), known from the scoring passes,
// so every wave forms p = 2^(x - M_h) in registers as its blocks stream in,
// and the four waves' sums share that reference (they add without rescaling).
// Scores, value metadata and codes of a wave's next block load while the
// current one is accumulated; the value tiles are read once per step, through
// non-temporal loads (the metadata rows, shared by the two channel halves,
// through ordinary ones).
// FV: blocks with FP16 values may occur (a step whose controller promoted
// values); without it the kernel has no FP16-value path and none of its LDS.
template <int D, int CB, int NP, bool FV>
struct alignas(16) DecLds {
  int8_t As[2 * NP][D / VGROUP / 2][16 * 80];    // A operand per wave and value group
  float pt[FV ? 2 * NP : 1][FV ? BLOCK : 1][4];  // p of an FP16-value block per token
  float fsum[FV ? 2 * NP : 1][4][FV ? D : 1];    // the FP16-value blocks' sums per wave
  float sl[2 * NP][4];
};

// One chunk (sequence i, KV head g, chunk ch) on 2 NP waves: tid = the
// thread's index among them.  Every thread of the workgroup reaches the same
// two barriers (a workgroup of two such thread sets runs two chunks); a set
// with live = false computes its chunk and stores nothing.  RL != nullptr (a
// step whose INT8 pass stored no ŝ′): each wave first computes ŝ′ of its own
// blocks outside U (q16, C: the query and its scale, as the pass), so the
// scores it reads next are its own stores (RL: one area per wave).
template <int D, int CB, int NP, bool FV>
__device__ inline void decode_chunk(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab,
                                    int layer, int i, int g, int ch, bool live, int tid,
                                    DecLds<D, CB, NP, FV> &L, const uint16_t *q16 = nullptr,
                                    float C = 0.0f, RescoreLds<D> *RL = nullptr) {
  constexpr int NT = D / 16;                     // 16-channel tiles
  constexpr int NG = D / VGROUP;                 // value groups (two tiles each)
  constexpr int NTW = NT / 2, NGW = NG / 2;      // tiles and groups of one wave
  constexpr int AST = 80;                        // LDS row stride of A (bank spread)
  constexpr int NW = 2 * NP;                     // waves
  constexpr int PW = CB / NP;                    // blocks per wave
  constexpr int MR = (CB + 15) / 16;             // block maxima per lane
  static_assert(CB <= 64 && CB % NP == 0, "block flags sit in one 64-lane ballot");
  const int T = tab.T[i], NB = (T + BLOCK - 1) / BLOCK;
  // chunk ch of nch: blocks [ch NB / nch, (ch + 1) NB / nch), at most CB
  const int nch = tab.nch[i];
  const int b0 = (int)((long long)ch * NB / nch);
  const size_t ig = (size_t)i * s.Hkv + g;
  const int G = s.G;
  const int b1 = (int)((long long)(ch + 1) * NB / nch);
  const int nblk = b1 - b0;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hl = lane >> 4;                      // head of this lane in the MFMA output
  const int half = wave & 1, pair = wave >> 1;   // channel half, block residue mod NP
  const size_t u = unit_of(s, tab.slot[i], layer, g);
  const uint8_t *U = w.U + ig * s.NBmax;
  const uint8_t *V = w.V + ig * s.NBmax;

  auto &As = L.As;
  auto &pt = L.pt;
  auto &fsum = L.fsum;
  auto &sl = L.sl;
  // the chunk's block flags and both kinds of block maxima load at once
  // (no load waits on another); the first blocks' value metadata and codes
  // go out before the flags are used
  const int k16 = lane & 15;
  const size_t om = ((size_t)i * s.Hq + g * G + min(hl, G - 1)) * s.NBmax + b0;
  float m16v[MR], mhv[MR];                       // blocks 16 r + k of the chunk
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    m16v[r] = w.m16[om + min(16 * r + k16, nblk - 1)];
    mhv[r] = w.mhat[om + min(16 * r + k16, nblk - 1)];
  }
  const uint8_t uf = U[b0 + min(lane, nblk - 1)], vf = V[b0 + min(lane, nblk - 1)];
  // set once the flags are in: the chunk's U and V masks, and the chunk
  // reference per head (max over the chunk's blocks of the block maxima in
  // use; lane 16 h + k holds head h's maxima of blocks b0 + 16 r + k)
  unsigned long long umask = 0ull, vmask = 0ull;
  float Mh[4];
  float acc[NTW];
#pragma unroll
  for (int k = 0; k < NTW; ++k) acc[k] = 0.0f;
  float offacc[4][NGW];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int j = 0; j < NGW; ++j) offacc[h][j] = 0.0f;
  float lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const uint16_t *sv = w.stage_v + ig * s.Tmax * D;

  // A wave's block in flight: scores of the four heads, its groups' value
  // metadata of its token, its code tiles.  Loads are unconditional at
  // clamped indices (token T - 1, head G - 1); masks apply at use.
  struct Stage {
    float x[4];
    uint32_t meta[NGW];
    u32x2 pk[NTW];
  };
  // value metadata and codes (no flag needed), then the scores (FP16 keys'
  // on blocks of U, INT8 keys' elsewhere)
  // addresses: a wave-uniform base per block (and head) plus a 32-bit lane
  // offset, so the loads take their base from scalar registers
  auto fetch_vm = [&](Stage &st, int bb) {
    // the lane's token, clamped (bb is a block of the sequence: in [0, 64))
    const uint32_t tl = (uint32_t)min(lane, T - 1 - bb * BLOCK) & (BLOCK - 1);
    // the two channel halves' waves read the two halves of each token's
    // metadata row: ordinary loads, so that the second reader finds the
    // lines in L2 (non-temporal loads fetched them from HBM twice)
    const uint32_t *mp = t.vmeta + (u * s.Tmax + (size_t)bb * BLOCK) * NG + half * NGW;
    if constexpr (NGW == 2) {
      const u32x2 m = *(const u32x2 *)(mp + tl * (uint32_t)NG);
      st.meta[0] = m.x, st.meta[1] = m.y;
    } else {
      st.meta[0] = mp[tl * (uint32_t)NG];
    }
    const u32x2 *vc = (const u32x2 *)(t.vcodes + (u * s.NBmax + bb) * (size_t)(32 * D)) + half * NTW * 64;
#pragma unroll
    for (int k = 0; k < NTW; ++k) st.pk[k] = __builtin_nontemporal_load(vc + (uint32_t)(k * 64 + lane));
  };
  auto fetch_sc = [&](Stage &st, int bb, unsigned long long umask) {
    const uint32_t tl = (uint32_t)min(lane, T - 1 - bb * BLOCK) & (BLOCK - 1);
    const bool up = __builtin_amdgcn_readfirstlane((int)((umask >> (bb - b0)) & 1ull)) != 0;
    const float *src = (up ? w.sp : w.shat) + ((size_t)i * s.Hq + g * G) * s.Tmax + (size_t)bb * BLOCK;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      // the head's row base pinned to scalar registers (without it the
      // compiler adds the head offsets to the per-lane address in 64 bits)
      const uint64_t a = (uint64_t)(src + (size_t)min(h, G - 1) * s.Tmax);
      typedef const __attribute__((address_space(1))) float gfloat;
      gfloat *sh = (gfloat *)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                              (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a));
      st.x[h] = sh[tl];
    }
  };
  // quantized values: p*s as fixed point against the INT4 codes
  // byte selectors of the quad transpose (v_perm: bytes 0-3 from the second
  // operand, 4-7 from the first): lanes with bit 0 clear take [x0 y0 x2 y2],
  // set [y1 x1 y3 x3]; then bit 1 clear [x0 x1 z0 z1], set [z2 z3 x2 x3]
  const uint32_t qsel1 = (lane & 1) ? 0x03070105u : 0x06020400u;
  const uint32_t qsel2 = (lane & 2) ? 0x03020706u : 0x05040100u;
  auto body = [&](const Stage &cur, int b) {
    const bool valid = b * BLOCK + lane < T;
    float sc[NGW], of[NGW];
    uint32_t ex = 0;
#pragma unroll
    for (int j = 0; j < NGW; ++j) {
      const uint32_t m = valid ? cur.meta[j] : 0u;
      sc[j] = h2f((uint16_t)(m & 0xffffu));
      of[j] = h2f((uint16_t)(m >> 16));
      ex = max(ex, __builtin_amdgcn_ubfe(m, 10, 5));   // binary16 exponent field of the scale
    }
    // E = the largest exponent field in the block (this wave's groups), by
    // bisection on ballots; every scale is below 2^(E - 14), so with
    // e = E - 36 and p <= 1 each A = rint(p s 2^-e) is below 2^22 (22 bits
    // relative to the block's largest scale), and 2^-e, 2^e, 2^(e + 16) are
    // normal floats (E in [0, 30])
    int E = 0;
#pragma unroll
    for (int bit = 4; bit >= 0; --bit)
      if (__ballot(ex >= (uint32_t)(E | (1 << bit)))) E |= 1 << bit;
    const float fm = __int_as_float((163 - E) << 23);          // 2^-e
    const float f0 = __int_as_float((E + 91) << 23);           // 2^e
    const float f2 = __int_as_float((E + 107) << 23);          // 2^(e + 16)
    float p[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      p[h] = (valid && h < G) ? __builtin_amdgcn_exp2f(cur.x[h] - Mh[h]) : 0.0f;
      lsum[h] += p[h];
    }
#pragma unroll
    for (int j = 0; j < NGW; ++j) {
      int8_t *Aj = As[wave][j];
      const float sce = sc[j] * fm;              // exact: a power-of-two scaling
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        offacc[h][j] = fmaf(p[h], of[j], offacc[h][j]);
        // A + 0x808080 with A = rint(p s 2^-e) in [0, 2^22) (p, s >= 0), in
        // one rounding: a float in [2^23, 2^24), where the spacing is 1, so
        // its bits are 0x4B000000 | (A + 0x8080).  One XOR then leaves three
        // signed bytes L0 + 2^8 L1 + 2^16 L2 = A, each in [-128, 127], and a
        // zero fourth byte (the same bytes as (A + 0x808080) ^ 0x808080)
        const uint32_t Bv = __float_as_uint(fmaf(p[h], sce, 8421504.0f)) ^ 0x4B008080u;
        // 4 x 4 byte transpose inside each quad of lanes (tokens 4 m .. 4 m + 3):
        // lane 4 m + l then holds limb l of the four tokens, one dword of row
        // 4 h + l (row 4 h + 3 gets the zero bytes)
        const uint32_t y1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)Bv, 0xB1, 0xf, 0xf, false);
        const uint32_t x1 = __builtin_amdgcn_perm(y1, Bv, qsel1);
        const uint32_t y2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)x1, 0x4E, 0xf, 0xf, false);
        const uint32_t x2 = __builtin_amdgcn_perm(y2, x1, qsel2);
        *(uint32_t *)&Aj[(h * 4 + (lane & 3)) * AST + (lane & ~3)] = x2;
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < NGW; ++j) {
      const v4i Aop = *(const v4i *)&As[wave][j][(lane & 15) * AST + 16 * (lane >> 4)];
#pragma unroll
      for (int k = 2 * j; k < 2 * j + 2; ++k) {
        v4i Bop;
        Bop[0] = (int)(cur.pk[k].x & 0x0f0f0f0fu);
        Bop[1] = (int)((cur.pk[k].x >> 4) & 0x0f0f0f0fu);
        Bop[2] = (int)(cur.pk[k].y & 0x0f0f0f0fu);
        Bop[3] = (int)((cur.pk[k].y >> 4) & 0x0f0f0f0fu);
        const v4i Dm = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aop, Bop, (v4i){0, 0, 0, 0}, 0, 0, 0);
        // rows 4 h + 0..2 hold head h's limb sums (each below 2^17 in
        // magnitude), row 4 h + 3 is zero; limbs 0 and 1 recombine in int32
        // (below 2^26: one rounding of 2^-24 relative in the conversion)
        const int D01 = Dm[0] + (Dm[1] << 8);
        acc[k] = fmaf((float)Dm[2], f2, fmaf((float)D01, f0, acc[k]));
      }
    }
    wave_lds_sync();
  };
  // FP16 values of a promoted block (rung 2): plain fp32 accumulation.  The
  // wave forms p for the block's 64 tokens (lane = token) like the quantized
  // path, then takes its half of the tokens with lane = CPL consecutive
  // channels, so each token's values are one coalesced row load, and keeps
  // per-head sums of its own (added to the chunk's sums at the end)
  constexpr int CPL = D / 64;                    // channels per lane on this path
  float fa[4][CPL];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int c = 0; c < CPL; ++c) fa[h][c] = 0.0f;
  auto body_fp16 = [&](int b) {
    if constexpr (!FV) return;
    const int tk = min(b * BLOCK + lane, T - 1);
    const bool valid = b * BLOCK + lane < T;
    const bool up = (umask >> (b - b0)) & 1ull;
    const float *src = (up ? w.sp : w.shat) + ((size_t)i * s.Hq + g * G) * s.Tmax + tk;
    float p4[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float x = src[(size_t)min(h, G - 1) * s.Tmax];
      p4[h] = (valid && h < G) ? __builtin_amdgcn_exp2f(x - Mh[h]) : 0.0f;
      lsum[h] += p4[h];
    }
    *(float4 *)&pt[wave][lane][0] = make_float4(p4[0], p4[1], p4[2], p4[3]);
    wave_lds_sync();
    // rows past T carry p = 0 and load row T - 1 (the staging past T is not
    // written); sixteen rows' loads go out together
    const int nlast = min(BLOCK, T - b * BLOCK) - 1;
    const uint16_t *col = sv + (size_t)b * BLOCK * D + CPL * lane;
    for (int r0 = BLOCK / 2 * half; r0 < BLOCK / 2 * (half + 1); r0 += 16) {
      uint32_t xr[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint16_t *e = col + (size_t)min(r0 + j, nlast) * D;
        xr[j] = CPL == 2 ? *(const uint32_t *)e : (uint32_t)*e;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float4 pr = *(const float4 *)&pt[wave][r0 + j][0];
        const float pq[4] = {pr.x, pr.y, pr.z, pr.w};
        float v[CPL];
        v[0] = h2f((uint16_t)(xr[j] & 0xffffu));
        if constexpr (CPL == 2) v[CPL - 1] = h2f((uint16_t)(xr[j] >> 16));
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
          for (int c = 0; c < CPL; ++c) fa[h][c] = fmaf(pq[h], v[c], fa[h][c]);
      }
    }
    wave_lds_sync();
  };
  // fully unrolled over the wave's blocks, so the two stages keep fixed
  // registers and each wait covers only the older stage's loads; blocks with
  // FP16 values are skipped here and accumulated afterwards
  Stage st[2];
  if (RL != nullptr && live) {
    // this wave's blocks outside U, before any stage register is taken (so
    // the value loads wait for the flags here).  Both channel halves of a
    // block compute and store the same bits, and each reads the scores only
    // after its own stores: whichever store lands last, the bits it reads
    // are its own results
    const unsigned long long outside = ~__ballot(lane < nblk && uf != 0) & (nblk >= 64 ? ~0ull : (1ull << nblk) - 1ull);
    if (outside)
      for (int k = pair; k < nblk; k += NP)
        if ((outside >> k) & 1ull) rescore_block<D, false>(s, t, w, tab, layer, q16, C, i, g, b0 + k, RL[wave]);
  }
  fetch_vm(st[0], min(b0 + pair, b1 - 1));
  if (PW > 1) fetch_vm(st[1], min(b0 + pair + NP, b1 - 1));
  umask = __ballot(lane < nblk && uf != 0);
  vmask = FV ? __ballot(lane < nblk && vf != 0) : 0ull;
  {
    float bmv = -INFINITY;
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const int k = 16 * r + k16;
      if (hl < G && k < nblk) bmv = fmaxf(bmv, ((umask >> k) & 1ull) ? m16v[r] : mhv[r]);
    }
    const float bm = bfly_max<16>(bmv);
#pragma unroll
    for (int h = 0; h < 4; ++h)
      Mh[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bm), 16 * h));
  }
  fetch_sc(st[0], min(b0 + pair, b1 - 1), umask);
  if (PW > 1) fetch_sc(st[1], min(b0 + pair + NP, b1 - 1), umask);
#pragma unroll
  for (int q = 0; q < PW; ++q) {
    const int bb = b0 + pair + NP * q;
    if (bb >= b1) break;
    if (!((vmask >> (bb - b0)) & 1ull)) body(st[q & 1], bb);
    __builtin_amdgcn_sched_barrier(0);
    if (q + 2 < PW && bb + 2 * NP < b1) {       // (a shorter chunk loads nothing twice)
      fetch_vm(st[q & 1], bb + 2 * NP);
      fetch_sc(st[q & 1], bb + 2 * NP, umask);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (FV && vmask) {
    for (int bb = b0 + pair; bb < b1; bb += NP)
      if ((vmask >> (bb - b0)) & 1ull) body_fp16(bb);
    if constexpr (FV) {
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int c = 0; c < CPL; ++c) fsum[wave][h][CPL * lane + c] = fa[h][c];
    }
  }

  // offset terms: head h, group j summed over the wave's tokens; channel
  // tile k belongs to group k / 2
  float offs[4][NGW];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int j = 0; j < NGW; ++j) offs[h][j] = bfly_sum<64>(offacc[h][j]);
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    const float o = hl == 0 ? offs[0][k / 2] : hl == 1 ? offs[1][k / 2] : hl == 2 ? offs[2][k / 2] : offs[3][k / 2];
    acc[k] += o;
  }
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float lv = bfly_sum<64>(lsum[h]);
    if (lane == 0) sl[wave][h] = lv;
  }
  // the NP block residues' sums (same reference M_h) add in LDS, in the A
  // area, in residue order; the softmax sums come from the waves of channel
  // half 0
  __syncthreads();
  float *red = (float *)&As[0][0][0];            // [NW waves][NTW][64]
  static_assert(sizeof(As) >= NW * NTW * 64 * sizeof(float), "merge fits in the A area");
#pragma unroll
  for (int k = 0; k < NTW; ++k) red[(wave * NTW + k) * 64 + lane] = acc[k];
  __syncthreads();
  for (int e = tid; e < NT * 64; e += 128 * NP) {
    const int k = e / 64, ln = e % 64, h = ln >> 4;
    const int hf = k / NTW, kk = k % NTW;        // waves 2 p + hf, residue p
    if (h < G && live) {
      float v = red[(hf * NTW + kk) * 64 + ln];
#pragma unroll
      for (int p = 1; p < NP; ++p) v += red[((2 * p + hf) * NTW + kk) * 64 + ln];
      if (FV && vmask) {                         // and every wave's FP16-value sums
        if constexpr (FV) {
#pragma unroll
          for (int q = 0; q < NW; ++q) v += fsum[q][h][k * 16 + (ln & 15)];
        }
      }
      float *part = w.part + ((ig * s.nchmax + ch) * G + h) * (size_t)(D + 2);
      part[k * 16 + (ln & 15)] = v;
    }
  }
  if (tid < G && live) {
    const int h = tid;
    float *part = w.part + ((ig * s.nchmax + ch) * G + h) * (size_t)(D + 2);
    part[D] = h == 0 ? Mh[0] : h == 1 ? Mh[1] : h == 2 ? Mh[2] : Mh[3];
    float l = sl[0][h];
#pragma unroll
    for (int p = 1; p < NP; ++p) l += sl[2 * p][h];
    part[D + 1] = l;
  }
}

}  // namespace kvq
