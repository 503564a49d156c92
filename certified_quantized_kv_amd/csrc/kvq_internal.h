// kvq_internal.h -- context layout and kernel argument blocks of libkvq.
//
// Layout of everything the library keeps in device memory (tier 1 and the
// per-step scratch) and of tier 2 in pinned host memory.  A "unit" is one
// (slot, layer, KV head); u = (slot * n_layers + layer) * n_kv_heads + g.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>
#include <tuple>

#include "../../include/kvq.h"

namespace kvq {

constexpr int MAX_CALL = KVQ_MAX_CALL_SEQS;
constexpr int MAX_NB = 4096;        // blocks per sequence (262144 tokens)
constexpr int DEC_CB = 8;           // blocks per split-K chunk of the dense decode kernels
constexpr int MIX_CB = 48;          // most blocks per split-K chunk of the mixed decode
static_assert(MIX_CB >= DEC_CB, "chunk partials are sized for DEC_CB");

// Tier 1, per unit (device memory):
//   kcodes [NBmax][64*d] u8   block-local MFMA operand order: the 16 bytes at
//                             ((ks*4 + nt)*64 + l)*16 are the codes of token
//                             nt*16 + l%16, channels ks*64 + 16*(l/16) + 0..15,
//                             each stored as code ^ 0x80 (= code - 128 as a
//                             signed byte)
//   kmeta  [NBmax][d]    u32  binary16 scale (low half), offset (high half)
//   vcodes [NBmax][32*d] u8   block-local MFMA operand order: for 16-channel
//                             tile nt and lane l, 8 bytes at (nt*64 + l)*8 hold
//                             the codes of channel nt*16 + l%16 for tokens
//                             16*(l/16) + p, p = 0..15: byte 4*(p/8) + p%4,
//                             high nibble when (p/4) is odd (see vnib())
//   vmeta  [Tmax][d/32]  u32  binary16 scale (low), offset (high) per group
//   eta    [NBmax]       f32  per-block value error annotation
//   vmin/vmax [d]        u32  order-mapped floats, running over all tokens
//   openk  [2][64][d]    u16  FP16 keys of the open (partial) block, two
//                             halves: an append reads the half its parity
//                             names and writes the other (see k_append)
//   kres   [Tmax][d]     u16  with resident keys: every FP16 key (written on
//                             append; the FP16 key staging of the unit)
// Tier 2, per unit (pinned host, device-mapped): t2k/t2v [Tmax][d] fp16.
struct Tier1 {
  uint8_t *kcodes;
  uint32_t *kmeta;
  uint8_t *vcodes;
  uint32_t *vmeta;
  float *eta;
  uint32_t *vmin, *vmax;
  uint16_t *openk;
  uint16_t *t2k, *t2v;     // device-mapped pointers to pinned host memory
  uint16_t *kres;          // resident FP16 keys [unit][Tmax][d], or null
};

// Per-step scratch, indexed by the position i of a sequence in the call.
struct Step {
  float *qp;                       // [B][Hq][d]
  float *shat, *sp;                // [B][Hq][Tmax]
  float *mhat, *delta, *m16;       // [B][Hq][NBmax]
  uint32_t *Lhat, *L16, *What, *pi, *Wt, *W16;
  uint8_t *vh;                     // [B][Hq][NBmax]
  int32_t *k0, *ssize;             // [B][Hq]
  unsigned long long *ssd;         // [B][Hq]
  double *ekey64, *eval64;         // [B][Hq]
  unsigned long long *evs;         // [B][Hq][2] E_val numerator (no value promoted), denominator
  uint32_t *hflags;                // [B][Hq]
  int8_t *hlevel;                  // [B][Hq]
  uint8_t *U, *Knew, *V;           // [B][Hkv][NBmax]
  uint32_t *gstat;                 // [B][Hkv] bit0 done, bit1 any rung 3
  uint32_t *runs;                  // [B][Hkv][2][RUNMAX] start | len << 16 (scratch)
  unsigned long long *plan;        // runs for the host (layout at emit_runs)
  uint16_t *stage_k, *stage_v;     // [B][Hkv][Tmax][d] ([units][Tmax][d] keys when resident)
  float *part, *partd;             // [B][Hkv][NCH][G][d + 2]
  uint8_t *gdense;                 // [B][Hkv]
  uint32_t *rlist;                 // [B * Hkv * NBmax] units whose ŝ′ a step rescores
};

struct SeqTab {
  int n;
  int slot[MAX_CALL];
  int T[MAX_CALL];
  int nbc[MAX_CALL + 1];            // nbc[i] = blocks of the sequences before i
  int nch[MAX_CALL];                // split-K chunks of sequence i in the mixed decode
};

struct Shape {
  int L, Hq, Hkv, G, d, Tmax, NBmax, runmax, nchmax, B;
  int ncu;                          // compute units of the device
  int kres;                         // 1: FP16 key staging per unit, kept across steps
};

// Arguments of the dense comparator: FP16 q [n][Hq][d], K and V
// [n][tcap][Hkv][d] in device memory, T[i] tokens of sequence i.
struct DenseArgs {
  int n;
  int T[MAX_CALL];
  long long tcap;
  const uint16_t *q, *k, *v;
};

struct Thresh {
  int tau_ppm, rho_ppm, R1, frac_ppm;
  double eps_key, v_tol;
  int force_dense;
  int fp16_values;                  // every block's values from tier 2 (ablation)
};

// Layout helpers (host and device).
__host__ __device__ inline size_t unit_of(const Shape &s, int slot, int layer, int g) {
  return ((size_t)slot * s.L + layer) * s.Hkv + g;
}

// Index (in units of Tmax rows) of the FP16 key staging of call position i,
// KV head g: one area per call position, or, with resident keys, one per
// unit so that promoted blocks stay valid across steps.
__host__ __device__ inline size_t stage_k_area(const Shape &s, int i, int g, int slot, int layer) {
  return s.kres ? unit_of(s, slot, layer, g) : (size_t)i * s.Hkv + g;
}

// Capacity (entries) of each of the K and V halves of the promotion plan:
// the selection lists runs per query head.
__host__ __device__ inline size_t plan_kcap(const Shape &s) {
  return (size_t)s.B * s.Hq * s.runmax;
}

// Byte (within a block's value codes) and nibble shift of (row r, channel c).
// Unpacking a lane's 8 bytes as (x & 0x0f0f0f0f), (x >> 4) & 0x0f0f0f0f per
// dword yields its 16 tokens in order.
__host__ __device__ inline void vnib(int r, int c, int &byte, int &shift) {
  const int nt = c >> 4, l = (c & 15) + 16 * (r >> 4), p = r & 15;
  byte = (nt * 64 + l) * 8 + (p >> 3) * 4 + (p & 3);
  shift = ((p >> 2) & 1) * 4;
}

// ---- kernel launch with optional per-kernel timing ------------------------------
// While a timing category is open on the calling thread, every launch gets
// its own pair of events that the runtime stamps with the kernel's start and
// end (hipExtLaunchKernel), so a pair's elapsed time is that one kernel's
// duration on its stream.
struct KernelClock {
  hipEvent_t *ev;      // 2 * cap events
  int cap, used;
  int open;            // category of launches being timed, -1 when none
  int cat[64];
};
KernelClock *&kernel_clock();      // thread-local; defined in kvq_api.hip

template <typename... P, typename... A>
inline hipError_t launch_k(void (*k)(P...), dim3 grid, dim3 block, uint32_t shmem,
                           hipStream_t st, A... a) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> args{a...};
  hipEvent_t e0 = nullptr, e1 = nullptr;
  KernelClock *kc = kernel_clock();
  if (kc && kc->open >= 0 && kc->used < kc->cap) {
    e0 = kc->ev[2 * kc->used];
    e1 = kc->ev[2 * kc->used + 1];
    kc->cat[kc->used++] = kc->open;
  }
  hipError_t e = std::apply(
      [&](auto &...x) {
        void *ptrs[] = {(void *)&x...};
        return hipExtLaunchKernel((const void *)k, grid, block, ptrs, shmem, st, e0, e1, 0);
      },
      args);
  return e != hipSuccess ? e : hipGetLastError();
}

// ---- launchers (each in its own .hip file) ---------------------------------

struct AppendArgs {
  int n, layer;
  int slot[MAX_CALL], T_old[MAX_CALL], n_new[MAX_CALL], in_off[MAX_CALL], n_blk[MAX_CALL];
  int par[MAX_CALL];                // half of openk holding the open block's keys
};
hipError_t launch_append(const Shape &s, const Tier1 &t, const AppendArgs &a, const uint16_t *k,
                         const uint16_t *v, int max_blk, hipStream_t st);

hipError_t launch_score_int8(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab,
                             int layer, const uint16_t *q, float C, bool store, hipStream_t st);
// ŝ′ of the listed units (ig << 16 | block), after a pass that stored none.
hipError_t launch_rescore_int8(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab,
                               int layer, const uint16_t *q, float C, const uint32_t *list, int count,
                               hipStream_t st);
hipError_t launch_select(const Shape &s, const Step &w, const SeqTab &tab, int tau_ppm, int maxNB,
                         hipStream_t st);
hipError_t launch_score_fp16(const Shape &s, const Step &w, const SeqTab &tab, int layer,
                             int maxNB, hipStream_t st);
hipError_t launch_control(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab,
                          int layer, const Thresh &th, int round, int maxNB, hipStream_t st);
// rcount > 0: extra workgroups compute ŝ′ of rlist's blocks (as
// launch_rescore_int8) beside the evaluation
hipError_t launch_eval(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab, int layer,
                       const Thresh &th, int maxNB, const uint16_t *q, float C, const uint32_t *rlist,
                       int rcount, hipStream_t st);
hipError_t launch_decide(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab,
                         int layer, const Thresh &th, int round, int maxNB, hipStream_t st);
hipError_t launch_finalize(const Shape &s, const Step &w, const SeqTab &tab, const Thresh &th,
                           float *e_key, float *e_val, int8_t *level, hipStream_t st);
hipError_t launch_decode(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab,
                         int layer, bool values, hipStream_t st);
hipError_t launch_dense_staged(const Shape &s, const Step &w, const SeqTab &tab, int layer,
                               const uint16_t *q16, int maxNB, hipStream_t st);
// mode 0: partials chosen by each head's level; 1: mixed partials; 2: dense;
// 3: mixed partials, and the outputs of a first round that flagged no head.
// fused_extra >= 0: the mixed partials came from k_eval_decode launched with
// that many workgroups beside its decode workgroups (its chunking), else -1.
hipError_t launch_combine(const Shape &s, const Step &w, const SeqTab &tab, float *out, int mode,
                          float *e_key, float *e_val, int8_t *level, int fused_extra, hipStream_t st);
// Split-K chunks per sequence of the mixed decode (tab.nch), for workgroups of
// per_wg chunks beside `extra` other workgroups of the same launch.
void mix_chunk_counts(const Shape &s, SeqTab &tab, int cb, int per_wg, int extra);
// The first controller round and the speculative mixed decode in one launch
// (k_eval_decode): the heads' evaluation beside the decode's chunks, two per
// workgroup.  resc: the step's INT8 pass stored no ŝ′; the decode computes
// those of the blocks outside U itself (q, C: the query and its scale).
// Sets *extra to the number of evaluation workgroups (for launch_combine),
// or to -1 when the launch shape does not allow the fused launch (then
// nothing was launched).
hipError_t launch_eval_decode(const Shape &s, const Tier1 &t, const Step &w, const SeqTab &tab,
                              int layer, const Thresh &th, int maxNB, const uint16_t *q, float C,
                              bool resc, int *extra, hipStream_t st);
// Whether launch_eval_decode takes this call (else it launches nothing).
bool eval_decode_fits(const Shape &s, const SeqTab &tab);
hipError_t launch_dense_vram(const Shape &s, const Step &w, const DenseArgs &a, int maxNB,
                             hipStream_t st);
hipError_t launch_exp2k(const float *x, float *y, int64_t n, hipStream_t st);
hipError_t launch_selftest_sort(const unsigned long long *in, int n, unsigned long long *out, int *path,
                                hipStream_t st);
hipError_t launch_export_kcodes(const Shape &s, const Tier1 &t, size_t u, int T, uint8_t *dst,
                                hipStream_t st);
hipError_t launch_export_vcodes(const Shape &s, const Tier1 &t, size_t u, int T, uint8_t *dst,
                                hipStream_t st);
const char *noalloc_last_error();   // kvq_noalloc.hip
void set_score_grid_cap(int wgs);   // kvq_score.hip (test hook)
void set_mix_chunk_blocks(int cb);  // kvq_decode.hip (test hook)
int mix_chunk_blocks();
hipError_t launch_copy_blocks(const uint32_t *list, int n, const uint16_t *src, uint16_t *dst,
                              int d, hipStream_t st);

}  // namespace kvq
