// kvq_score.hip -- the INT8 scoring pass and the FP16 scoring of promoted
// blocks ("Runtime-Certified Bounded-Error Quantized Attention",
// Méthodologie §3: a lightweight pass over the INT8 keys estimates per-block
// attention mass; Méthodologie §2: the per-token score perturbation Delta
// that bounds the key error, from quantization scales and query values).
//
// Scores are in log2 units: q'_c = fl32(q_c * fl32(log2(e) / sqrt(d))).
//
// INT8 score of token t in block b for query head h (exact integer core):
//   a_c = fl32(q'_c s_bc),  e = ilogb(max_c |a_c|) - 21,  A_c = rint(a_c 2^-e)
//   D_t = sum_c A_c (code_tc - 128)        (exact; any order)
//   beta = dot of q' with fl32(off + 128 s) in the fixed order below
//   shat_t = fmaf(fl32(D_t), 2^e, beta)
// The four query heads of a KV head share the block's codes, so the core is
// a real contraction: 16 rows (4 heads x 3 signed-byte limbs of A, + 1 zero
// row each) x 64 channels x 16 tokens per v_mfma_i32_16x16x64_i8.  Limbs:
// A = L2 2^16 + L1 2^8 + L0 with L0, L1 in [-128, 127]; each limb's dot
// product is exact in int32, and D_t is recombined exactly (in fp64, where
// it is below 2^38) before its one rounding to fp32.
//
// Per-block channel sums (beta and the Delta' sum): one fma chain from 0
// over the channels in ascending order, acc <- fmaf(x_c, y_c, acc).  A chain
// is sequential, so the wave runs its chains in batches: lane 4 h + k takes
// query head h of the batch's unit k (four consecutive blocks of one KV
// head), with the units' (off + 128 s, t_c) pairs and the group's q' rows
// staged in LDS.
//
// Delta'_b (bound on |shat_t - s'_t|, s' the FP16-key score below):
//   K'_c = max(|off_c|, |fmaf(256, s_c, off_c)|)
//   t_c  = fmaf(d 2^-22, K'_c, s_c / 2)
//   Delta' = fl32(fl32(sum_c |q'_c| t_c + R) (1 + 2^-15)), R = 64 d 2^e
// (s_c/2: quantization half-step; d 2^-22 K': fp32 evaluation of both score
// chains; R: rounding of A; the last factor: evaluation of Delta' itself.)
//
// FP16-key score (promoted blocks): s'_t = fma chain over c ascending of
// q'_c * k_tc from 0.  Block ingredients of any score row x:
//   m_b = max_t x_t,   L_b = sum_t floor(2^24 exp2k(fl32(x_t - m_b)))  (exact).
#include <algorithm>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_rescore.h"
#include "kvq_blockops.h"

namespace kvq {

typedef int v4i __attribute__((ext_vector_type(4)));

// Work split: a batch is up to four consecutive blocks of one (sequence, KV
// head), numbered sequence-major, then KV head, then block; wave k of the
// grid (W waves) takes batches k, k + W, k + 2W, ...  At any moment the grid
// streams one window of W consecutive batches, which keeps the HBM channels
// evenly loaded (measured faster than each wave sweeping a contiguous run
// of its own).  A batch's units share one query group: the group's q rows
// and the units' key metadata (contiguous in memory) are fetched together
// one batch ahead, a unit's codes one unit ahead.  Rows of the score tile
// above G repeat head 0, so every lane computes a value that is written
// somewhere valid: the stores carry no lane conditions, and the compiler's
// wait counts stay exact (a store under a lane condition makes it assume
// the store was skipped and wait for every older load).  The kernel also
// carries the step set-up (q' for the later kernels, flags cleared).  Codes
// and metadata are read once per step and the scores read once later: both
// go through non-temporal loads and stores, which leave the caches to the
// data that is reused.
// ST: the pass stores every block's INT8 scores ŝ′; without it only the
// block ingredients are stored, and the blocks that end up outside U get
// their ŝ′ after the selection (rescore_block, kvq_rescore.h: in the decode
// waves of a fused first round, in workgroups beside the heads' evaluation,
// or in k_rescore_int8).
template <int D, bool ST>
__global__ __launch_bounds__(256, 4) void k_score_int8(Shape s, Tier1 t, Step w, SeqTab tab, int layer,
                                                    const uint16_t *__restrict__ q16, float C) {
  constexpr int CW = D / 16;            // channels per lane-chunk
  constexpr int NKS = D / 64;           // MFMA k-steps per block
  constexpr int AST = D + 16;           // LDS row stride of the A operand (bank spread)
  constexpr int NBT = 4;                // units per batch
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int h = lane >> 4, jc = lane & 15;
  const int G = s.G;
  const int hs = h < G ? h : 0;         // head slot of the lane's row

  __shared__ __align__(16) int8_t As[4][16][AST];
  __shared__ __align__(16) uint16_t Ss[4][NBT][D];   // scales of the batch's units
  __shared__ __align__(16) float UTs[4][NBT][2 * D]; // (off + 128 s, t_c) per channel
  __shared__ __align__(16) float Qs[4][4][D];        // q' rows of the batch's group (head slots)
  __shared__ float2 Bs[4][NBT][4];                   // (beta, Delta' sum) per (unit, head slot)

  int NBA = 0;                          // batches of the call
  for (int ii = 0; ii < tab.n; ++ii) NBA += s.Hkv * ((tab.nbc[ii + 1] - tab.nbc[ii] + NBT - 1) / NBT);
  const int W = gridDim.x * 4;
  // workgroups go to the XCDs in turn: numbered so that each XCD takes one
  // contiguous range of batches, and the lines of the per-block arrays
  // written here fill up in one XCD's L2 (about 6 % less time at batch 4 than
  // with consecutive batches on different XCDs)
  const int nx = gridDim.x, bx = blockIdx.x;
  const int wid = ((nx % 8 == 0) ? (bx % 8) * (nx / 8) + bx / 8 : bx) * 4 + wave;
  // batch -> (sequence, KV head, first block, units); wave-uniform
  auto locate = [&](int bi, int &ii, int &gg, int &bb, int &nn) {
    ii = 0;
    int nbi = tab.nbc[1] - tab.nbc[0];
    int per = (nbi + NBT - 1) / NBT;
    while (bi >= s.Hkv * per) {
      bi -= s.Hkv * per;
      ++ii;
      nbi = tab.nbc[ii + 1] - tab.nbc[ii];
      per = (nbi + NBT - 1) / NBT;
    }
    gg = bi / per;
    bb = (bi - gg * per) * NBT;
    nn = min(NBT, nbi - bb);
  };

  v4i Bn[NKS][4];                       // codes of the unit in flight
  uint32_t kb[CW];                      // metadata of the batch in flight (row h: unit h)
  uint32_t qb[CW / 2];                  // q slice (head slot h) of the batch in flight
  auto fetch = [&](int ii, int gg, int bb) {
    const size_t uu = unit_of(s, tab.slot[ii], layer, gg);
    const uint8_t *kc = t.kcodes + (uu * s.NBmax + bb) * (size_t)(BLOCK * D);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        Bn[ks][nt] = __builtin_nontemporal_load(
            (const v4i *)(kc + ((size_t)((ks * 4 + nt) * 64 + lane)) * 16));
  };
  auto fetch_meta = [&](int ii, int gg, int bb, int nn) {
    const size_t uu = unit_of(s, tab.slot[ii], layer, gg);
    const uint32_t *km = t.kmeta + (uu * s.NBmax + bb + min(h, nn - 1)) * D + jc * CW;
#pragma unroll
    for (int c = 0; c < CW; ++c) kb[c] = __builtin_nontemporal_load(&km[c]);
    const uint32_t *qs = (const uint32_t *)(q16 + ((size_t)ii * s.Hq + gg * G + hs) * D + jc * CW);
#pragma unroll
    for (int c = 0; c < CW / 2; ++c) qb[c] = qs[c];
  };

  float qv[CW];                         // q' of the lane's slice (head slot h)
  if (wid >= NBA) {
    step_setup(s, w, tab.n, q16, C, blockIdx.x * (size_t)blockDim.x + threadIdx.x,
               (size_t)gridDim.x * blockDim.x);
    return;
  }
  // the set-up's stores first, then the first batch's metadata and first
  // unit's codes, waited for in full: no wait count inside the loop has to
  // allow for a path from here
  step_setup(s, w, tab.n, q16, C, blockIdx.x * (size_t)blockDim.x + threadIdx.x,
             (size_t)gridDim.x * blockDim.x);
  int i, g, b, nbt;
  locate(wid, i, g, b, nbt);
  fetch_meta(i, g, b, nbt);
  fetch(i, g, b);
  __builtin_amdgcn_s_waitcnt(0);

  for (int bi = wid;;) {
    const bool more = bi + W < NBA;
    int ni = i, ng = g, nb = b, nn = nbt;
    if (more) locate(bi + W, ni, ng, nb, nn);
    // ---- the batch's set-up: scales, channel terms and q rows into LDS; the
    // next batch's metadata and q, and (past the first batch, whose codes
    // came with its metadata) the first unit's codes go out; then the
    // channel-sum chains (lane 4 h + k: head slot h of unit k)
    {
      uint32_t *srow = (uint32_t *)&Ss[wave][h][jc * CW];
      float *urow = &UTs[wave][h][2 * jc * CW];
      float *qrow = &Qs[wave][h][jc * CW];
#pragma unroll
      for (int c = 0; c < CW; c += 2) srow[c / 2] = (kb[c] & 0xffffu) | (kb[c + 1] << 16);
#pragma unroll
      for (int c = 0; c < CW; ++c) qv[c] = h2f((uint16_t)(qb[c / 2] >> (16 * (c % 2)))) * C;
#pragma unroll
      for (int c = 0; c < CW; c += 4) *(float4 *)&qrow[c] = make_float4(qv[c], qv[c + 1], qv[c + 2], qv[c + 3]);
#pragma unroll
      for (int c = 0; c < CW; c += 2) {
        float4 ut;
        float *e = (float *)&ut;
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const uint32_t m = kb[c + x];
          const float sv = h2f((uint16_t)(m & 0xffffu)), ov = h2f((uint16_t)(m >> 16));
          const float kp = fmaxf(fabsf(ov), fabsf(fmaf(256.0f, sv, ov)));
          e[2 * x] = fmaf(128.0f, sv, ov);
          e[2 * x + 1] = fmaf((float)D * 0x1p-22f, kp, 0.5f * sv);
        }
        *(float4 *)&urow[2 * c] = ut;
      }
    }
    if (more) fetch_meta(ni, ng, nb, nn);
    if (bi != wid) fetch(i, g, b);
    wave_lds_sync();
    if (lane < 4 * NBT) {
      const int kk = lane & (NBT - 1), hh = lane / NBT;
      const float *qrow = &Qs[wave][hh][0];
      const float *ut = &UTs[wave][kk][0];
      float beta = 0.0f, sd = 0.0f;
#pragma unroll 2
      for (int c4 = 0; c4 < D; c4 += 4) {
        const float4 qq = *(const float4 *)(qrow + c4);
        const float qw[4] = {qq.x, qq.y, qq.z, qq.w};
        float4 p[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) p[x] = *(const float4 *)&ut[2 * c4 + 4 * x];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float qf = qw[x];
          const float uc = (x % 2) ? p[x / 2].z : p[x / 2].x;
          const float tc = (x % 2) ? p[x / 2].w : p[x / 2].y;
          beta = fmaf(qf, uc, beta);
          sd = fmaf(fabsf(qf), tc, sd);
        }
      }
      Bs[wave][kk][hh] = make_float2(beta, sd);
    }
    wave_lds_sync();

    const int T = tab.T[i];
    const int hq = g * G + hs;
    // one unit of the batch; the first is a copy of its own, so that the
    // loop's wait counts allow for the stores of the previous unit between a
    // unit's codes and their use
    auto unit = [&](const int k) {
      const int bk = b + k;
      const int n = min(BLOCK, T - bk * BLOCK);

      // ---- prologue: exponent and limbs of A per head ---------------------------
      float sc4[CW];
      {
        const uint32_t *sp4 = (const uint32_t *)&Ss[wave][k][jc * CW];
        uint32_t sw[CW / 2];
        if constexpr (CW == 8) {
          const uint4 v = *(const uint4 *)sp4;
          sw[0] = v.x, sw[1] = v.y, sw[2] = v.z, sw[3] = v.w;
        } else {
          const uint2 v = *(const uint2 *)sp4;
          sw[0] = v.x, sw[1] = v.y;
        }
#pragma unroll
        for (int c = 0; c < CW; ++c) sc4[c] = h2f((uint16_t)(sw[c / 2] >> (16 * (c % 2))));
      }
      const float2 bd = Bs[wave][k][h];
      float a[CW];
      float am = 0.0f;
#pragma unroll
      for (int c = 0; c < CW; ++c) {
        a[c] = qv[c] * sc4[c];
        am = fmaxf(am, fabsf(a[c]));
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
        int8_t *row = &As[wave][h * 4][jc * CW];
#pragma unroll
        for (int c = 0; c < CW / 4; ++c) {
          ((uint32_t *)(row + 0 * AST))[c] = l0w[c];
          ((uint32_t *)(row + 1 * AST))[c] = l1w[c];
          ((uint32_t *)(row + 2 * AST))[c] = l2w[c];
          ((uint32_t *)(row + 3 * AST))[c] = 0u;
        }
      }
      const float pb = bd.x;
      // Delta' is stored with the block ingredients, after the contraction
      const float dv = (bd.y + (zero ? 0.0f : ldexpf(64.0f * (float)D, e))) * (1.0f + 0x1p-15f);
      wave_lds_sync();

      // ---- exact integer core on the matrix cores -------------------------------
      v4i acc[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt] = (v4i){0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const v4i Aop = *(const v4i *)&As[wave][lane & 15][ks * 64 + 16 * (lane >> 4)];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          acc[nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aop, Bn[ks][nt], acc[nt], 0, 0, 0);
        }
      }
      if (k + 1 < nbt) fetch(i, g, bk + 1);

      // ---- scores and block ingredients (lane: head slot lane/16, token lane%16)
      // D_t = 2^16 L2-sum + 2^8 L1-sum + L0-sum is exact in fp64 (below 2^38)
      const float sc = ldexpf(1.0f, e);
      float x[4];
      float mx = -INFINITY;
      float *dst = w.shat + ((size_t)i * s.Hq + hq) * s.Tmax + (size_t)bk * BLOCK;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const double Dd = fma((double)acc[nt][2], 65536.0, fma((double)acc[nt][1], 256.0,
                                                               (double)acc[nt][0]));
        x[nt] = fmaf((float)Dd, sc, pb);
        const bool ok = nt * 16 + jc < n;
        mx = ok ? fmaxf(mx, x[nt]) : mx;
        // tokens past T land inside the row's last block, which no reader
        // takes past T; rows above G write head 0's values again
        if constexpr (ST) __builtin_nontemporal_store(x[nt], &dst[nt * 16 + jc]);
      }
      mx = bfly_max<16>(mx);
      uint32_t Ls = 0u;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const uint32_t l = (uint32_t)floorf(0x1p24f * exp2k(x[nt] - mx));
        Ls += (nt * 16 + jc < n) ? l : 0u;
      }
      Ls = bfly_sum_u32<16>(Ls);
      {
        // every lane of a row holds its head's values: all store them
        const size_t o = ((size_t)i * s.Hq + hq) * s.NBmax + bk;
        w.mhat[o] = mx;
        w.Lhat[o] = Ls;
        w.delta[o] = dv;
      }
      wave_lds_sync();
    };
    unit(0);
    for (int k = 1; k < nbt; ++k) unit(k);
    if (!more) break;
    bi += W;
    i = ni, g = ng, b = nb, nbt = nn;
  }
}

template <int D>
int grid_score_int8(const Shape &s) {
  static int per_cu = 0;
  if (per_cu == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_score_int8<D, true>, 256, 0) != hipSuccess ||
        nb < 1)
      nb = 1;
    per_cu = nb;
  }
  return per_cu * s.ncu;
}

// Workgroups: what the device holds at once, or one wave per batch, or fewer
// while a test has capped the grid (kvq_selftest_launch_shape): the grid
// decides which wave scores which block and which blocks share a batch of
// channel-sum chains, never a result.  Past three batches per resident wave
// every wave takes one batch and the dispatcher hands out the rest as waves
// finish (the saturated memory system serves waves unevenly): 91.8 -> 89.7 us
// at four 128K sequences; at two (two batches per wave) the resident grid
// is faster (52.6 against 56.0 us).
static int g_score_cap = 0;
void set_score_grid_cap(int wgs) { g_score_cap = wgs > 0 ? wgs : 0; }

static int int8_grid(int resident, int batches) {
  const int cap = batches > 12 * resident ? (batches + 3) / 4 : resident;
  const int g = std::max(1, std::min(cap, (batches + 3) / 4));
  return g_score_cap ? std::min(g, g_score_cap) : g;
}

hipError_t launch_score_int8(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab,
                             int layer, const uint16_t *q, float C, bool store, hipStream_t st) {
  int batches = 0;                      // four blocks of one (sequence, KV head) each
  for (int i = 0; i < tab.n; ++i) batches += s.Hkv * ((tab.nbc[i + 1] - tab.nbc[i] + 3) / 4);
  if (s.d == 128) {
    const int grid = int8_grid(grid_score_int8<128>(s), batches);
    return store ? launch_k(k_score_int8<128, true>, dim3(grid), dim3(256), 0, st, s, t, w, tab, layer, q, C)
                 : launch_k(k_score_int8<128, false>, dim3(grid), dim3(256), 0, st, s, t, w, tab, layer, q, C);
  }
  const int grid = int8_grid(grid_score_int8<64>(s), batches);
  return store ? launch_k(k_score_int8<64, true>, dim3(grid), dim3(256), 0, st, s, t, w, tab, layer, q, C)
               : launch_k(k_score_int8<64, false>, dim3(grid), dim3(256), 0, st, s, t, w, tab, layer, q, C);
}

// ---- ŝ′ of listed blocks (after a pass that stored none): kvq_rescore.h -------
template <int D>
__global__ __launch_bounds__(256) void k_rescore_int8(Shape s, Tier1 t, Step w, SeqTab tab, int layer,
                                                   const uint16_t *__restrict__ q16, float C,
                                                   const uint32_t *__restrict__ list, int count) {
  __shared__ RescoreLds<D> L[4];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  rescore_units<D>(s, t, w, tab, layer, q16, C, list, count, blockIdx.x * 4 + wave, gridDim.x * 4,
                   L[wave]);
}

hipError_t launch_rescore_int8(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab,
                               int layer, const uint16_t *q, float C, const uint32_t *list, int count,
                               hipStream_t st) {
  if (count <= 0) return hipSuccess;
  const int grid = std::max(1, std::min((count + 3) / 4, 4 * s.ncu));
  if (s.d == 128)
    return launch_k(k_rescore_int8<128>, dim3(grid), dim3(256), 0, st, s, t, w, tab, layer, q, C, list, count);
  return launch_k(k_rescore_int8<64>, dim3(grid), dim3(256), 0, st, s, t, w, tab, layer, q, C, list, count);
}

// ---- FP16-key scores of blocks promoted this round ------------------------------
// One workgroup per (sequence, KV head, F16_BPW blocks), four waves per
// block (one block per workgroup measured fastest); wave h = query head of
// the group, lane = token.  A block's FP16 keys
// are staged with 16-byte coalesced loads into LDS rows padded to d*2 + 16
// bytes (conflict-free 16-byte row reads); q' is read at wave-uniform
// addresses.  Each lane runs the canonical fma chain over channels in
// ascending order.  The staged keys are read once and the scores stored
// once (non-temporal loads and stores: no cache allocation for the stream).
constexpr int F16_BPW = 1;             // blocks per workgroup (4 waves each)

template <int D>
__global__ __launch_bounds__(256 * F16_BPW) void k_score_fp16(Shape s, Step w, SeqTab tab, int layer) {
  constexpr int RST = D + 8;            // LDS row stride in halves (d*2 + 16 bytes)
  const int i = blockIdx.z, g = blockIdx.y;
  const int T = tab.T[i], NB = (T + BLOCK - 1) / BLOCK;
  const int part = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);   // block of this thread
  const int tid = threadIdx.x & 255;
  const int wave = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 3), lane = threadIdx.x & 63;
  const int b = blockIdx.x * F16_BPW + part;
  uint8_t *flag = w.Knew + ((size_t)i * s.Hkv + g) * s.NBmax + b;
  const bool active = b < NB && *flag != 0;
  const int n = min(BLOCK, T - b * BLOCK);
  __shared__ __align__(16) uint16_t skall[F16_BPW][BLOCK * RST];
  uint16_t *sk = skall[part];

  // all 64 rows are loaded at once (rows past n of a partial block lie inside
  // the staging buffer; their results are masked below)
  constexpr int NL = BLOCK * D / 8 / 256;
  if (active) {
    const uint16_t *src =
        w.stage_k + (stage_k_area(s, i, g, tab.slot[i], layer) * s.Tmax + (size_t)b * BLOCK) * D;
    v4i v[NL];
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int idx = tid + 256 * k;
      v[k] = __builtin_nontemporal_load(
          (const v4i *)(src + (size_t)(idx / (D / 8)) * D + (idx % (D / 8)) * 8));
    }
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int idx = tid + 256 * k;
      *(v4i *)&sk[(idx / (D / 8)) * RST + (idx % (D / 8)) * 8] = v[k];
    }
  }
  __syncthreads();
  if (active && wave < s.G) {
    const int hq = g * s.G + wave;
    const float *q = w.qp + ((size_t)i * s.Hq + hq) * D;
    float acc = 0.0f;
    const uint16_t *row = &sk[lane * RST];
#pragma unroll 4
    for (int c = 0; c < D; c += 8) {
      const uint4 kk = *(const uint4 *)&row[c];
      acc = fmaf(q[c + 0], h2f((uint16_t)(kk.x & 0xffffu)), acc);
      acc = fmaf(q[c + 1], h2f((uint16_t)(kk.x >> 16)), acc);
      acc = fmaf(q[c + 2], h2f((uint16_t)(kk.y & 0xffffu)), acc);
      acc = fmaf(q[c + 3], h2f((uint16_t)(kk.y >> 16)), acc);
      acc = fmaf(q[c + 4], h2f((uint16_t)(kk.z & 0xffffu)), acc);
      acc = fmaf(q[c + 5], h2f((uint16_t)(kk.z >> 16)), acc);
      acc = fmaf(q[c + 6], h2f((uint16_t)(kk.w & 0xffffu)), acc);
      acc = fmaf(q[c + 7], h2f((uint16_t)(kk.w >> 16)), acc);
    }
    const bool valid = lane < n;
    if (valid)
      __builtin_nontemporal_store(acc, &w.sp[((size_t)i * s.Hq + hq) * s.Tmax + (size_t)b * BLOCK + lane]);
    const float mx = bfly_max<64>(valid ? acc : -INFINITY);
    uint32_t L = valid ? (uint32_t)floorf(0x1p24f * exp2k(acc - mx)) : 0u;
    L = bfly_sum_u32<64>(L);
    if (lane == 0) {
      const size_t o = ((size_t)i * s.Hq + hq) * s.NBmax + b;
      w.m16[o] = mx;
      w.L16[o] = L;
    }
  }
  __syncthreads();
  if (active && tid == 0) *flag = 0;
}

hipError_t launch_score_fp16(const Shape &s, const Step &w, const SeqTab &tab, int layer,
                             int maxNB, hipStream_t st) {
  dim3 grid((maxNB + F16_BPW - 1) / F16_BPW, s.Hkv, tab.n);
  if (s.d == 128)
    return launch_k(k_score_fp16<128>, grid, dim3(256 * F16_BPW), 0, st, s, w, tab, layer);
  return launch_k(k_score_fp16<64>, grid, dim3(256 * F16_BPW), 0, st, s, w, tab, layer);
}

// ---- test hook: the decision exponential on a vector ------------------------------
__global__ void k_exp2k(const float *x, float *y, int64_t n) {
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x)
    y[idx] = exp2k(x[idx]);
}
hipError_t launch_exp2k(const float *x, float *y, int64_t n, hipStream_t st) {
  return launch_k(k_exp2k, dim3(1024), dim3(256), 0, st, x, y, n);
}

}  // namespace kvq
