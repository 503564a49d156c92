// kvq_api.hip -- the C ABI (include/kvq.h): context, tiers, and the host
// orchestration of one certified decode step.
//
// Decode step ("Runtime-Certified Bounded-Error Quantized Attention",
// Méthodologie §1-§3), all on the caller's stream except the promotion
// copies, which run on the context's copy stream and are joined by events:
//   1. q' (log2 units); INT8 scoring pass with per-block Delta' and (m, L);
//   2. per query head top-K* selection; per KV head union -> key runs;
//   3. host round trip: runs of FP16 key blocks are copied from pinned tier 2
//      to the device staging buffer (hipMemcpyAsync, side stream);
//   4. FP16 scoring of the new blocks; controller round (ranking check,
//      E_key, rung 1 widening, and for groups that stop: rung 3, rung 2);
//      repeat 3-4 while some group widened (at most widen_rounds + 1 rounds);
//   5. value runs copied (rung 2); rung 4 and the per-head outputs; whole KV
//      heads copied for groups with a dense head;
//   6. split-K decode (mixed and dense) and the combine.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "kvq_device.h"
#include "kvq_internal.h"

using namespace kvq;

namespace kvq {
KernelClock *&kernel_clock() {
  static thread_local KernelClock *clock = nullptr;
  return clock;
}
}  // namespace kvq

// Device cache of FP16 key blocks (KVQ_FLAG_KEY_CACHE), managed on the host:
// a block (unit u, block b) has key u * NBmax + b.  Least recently used
// replacement over an intrusive list (head = most recent); a slot used by
// this call or within the last n_layers calls (one pass over the layers, so
// the same layer's previous step) is not evicted, so a working set larger
// than the cache keeps the cached part instead of cycling through it, and a
// miss of one KV head cannot evict a block another head of the same call is
// about to hit.
struct KeyCache {
  int64_t slots = 0;
  int64_t guard = 1;
  uint16_t *dev = nullptr;             // [slots][BLOCK][d]
  std::vector<int32_t> of;             // [unit * NBmax + b] -> slot, or -1
  std::vector<int64_t> owner;          // [slot] -> key, or -1
  std::vector<int64_t> used;           // [slot] call stamp of the last use
  std::vector<int32_t> prev, next;
  int32_t head = -1, tail = -1;
  std::vector<int32_t> free_slots;
  int64_t now = 0;
  uint32_t *list_host = nullptr;       // pinned [2][cap][2]: hits, then admissions
  uint32_t *list_dev = nullptr;        // device copy of the lists
  size_t cap = 0;                      // entries per list

  void unlink(int32_t x) {
    if (prev[x] >= 0) next[prev[x]] = next[x]; else head = next[x];
    if (next[x] >= 0) prev[next[x]] = prev[x]; else tail = prev[x];
    prev[x] = next[x] = -1;
  }
  void push_front(int32_t x) {
    prev[x] = -1;
    next[x] = head;
    if (head >= 0) prev[head] = x;
    head = x;
    if (tail < 0) tail = x;
  }
  void touch(int32_t x) {
    used[x] = now;
    unlink(x);
    push_front(x);
  }
  void drop(int64_t key) {
    const int32_t x = of[key];
    if (x < 0) return;
    of[key] = -1;
    owner[x] = -1;
    unlink(x);
    free_slots.push_back(x);
  }
  // a slot for `key`, or -1 when every slot is protected
  int32_t admit(int64_t key) {
    int32_t x = -1;
    if (!free_slots.empty()) {
      x = free_slots.back();
      free_slots.pop_back();
    } else if (tail >= 0 && used[tail] + guard <= now) {
      x = tail;
      of[owner[x]] = -1;
      unlink(x);
    } else {
      return -1;
    }
    owner[x] = key;
    of[key] = x;
    used[x] = now;
    push_front(x);
    return x;
  }
};

struct kvq_ctx {
  kvq_config cfg;
  KeyCache kc;
  Shape s;
  Thresh th;
  Tier1 t;
  Step w;
  uint16_t *t2k_host = nullptr, *t2v_host = nullptr;
  std::vector<int64_t> T;     // [slot][layer]
  std::vector<uint8_t> opar;  // [slot][layer] half of openk holding the open block
  std::vector<void *> dallocs;
  hipStream_t cstream = nullptr;
  hipEvent_t ev_start = nullptr, ev_copy = nullptr, ev_plan = nullptr, ev_spec = nullptr;
  hipEvent_t ev_k[128] = {};   // kernel timing pairs
  hipEvent_t ev_c[32] = {};    // copy timing pairs
  hipEvent_t ev_tot[2] = {};
  unsigned long long *plan_host = nullptr;
  uint8_t *u_host = nullptr;   // the call's group unions U after the selection
  uint32_t *rlist_host = nullptr;  // units outside U whose ŝ′ a deferred step rescores
  std::vector<int32_t> uppm;   // [layer] blocks in U at the last read, parts per million
  size_t plan_cap = 0;
  size_t plan_words = 0;
  int last_n = 0, last_layer = -1;
  int last_slot[MAX_CALL] = {}, last_T[MAX_CALL] = {};
  std::string err;
  int64_t dev_bytes = 0, host_bytes = 0;
  int device = 0;
};

namespace {

kvq_status fail(kvq_ctx *c, kvq_status st, const std::string &msg) {
  if (c) c->err = msg;
  return st;
}

#define HIPCK(ctx, expr)                                                             \
  do {                                                                               \
    hipError_t e_ = (expr);                                                          \
    if (e_ != hipSuccess)                                                            \
      return fail(ctx, KVQ_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

template <class P>
hipError_t dalloc(kvq_ctx *c, P **p, size_t bytes) {
  void *q = nullptr;
  hipError_t e = hipMalloc(&q, bytes ? bytes : 16);
  if (e != hipSuccess) return e;
  c->dallocs.push_back(q);
  c->dev_bytes += (int64_t)bytes;
  *p = (P *)q;
  return hipSuccess;
}

void free_all(kvq_ctx *c) {
  if (!c) return;
  (void)hipDeviceSynchronize();
  for (void *p : c->dallocs) (void)hipFree(p);
  c->dallocs.clear();
  if (c->t2k_host) (void)hipHostFree(c->t2k_host);
  if (c->t2v_host) (void)hipHostFree(c->t2v_host);
  if (c->plan_host) (void)hipHostFree(c->plan_host);
  if (c->u_host) (void)hipHostFree(c->u_host);
  if (c->rlist_host) (void)hipHostFree(c->rlist_host);
  if (c->kc.list_host) (void)hipHostFree(c->kc.list_host);
  if (c->cstream) (void)hipStreamDestroy(c->cstream);
  if (c->ev_start) (void)hipEventDestroy(c->ev_start);
  if (c->ev_copy) (void)hipEventDestroy(c->ev_copy);
  if (c->ev_plan) (void)hipEventDestroy(c->ev_plan);
  if (c->ev_spec) (void)hipEventDestroy(c->ev_spec);
  for (auto &e : c->ev_k)
    if (e) (void)hipEventDestroy(e);
  for (auto &e : c->ev_c)
    if (e) (void)hipEventDestroy(e);
  for (auto &e : c->ev_tot)
    if (e) (void)hipEventDestroy(e);
}

bool valid_seqs(const kvq_ctx *c, int n, const int32_t *ids) {
  if (n < 1 || n > c->cfg.max_batch || n > MAX_CALL || !ids) return false;
  for (int a = 0; a < n; ++a) {
    if (ids[a] < 0 || ids[a] >= c->cfg.max_batch) return false;
    for (int b = 0; b < a; ++b)
      if (ids[a] == ids[b]) return false;
  }
  return true;
}

// Step timing.  Kernels: while a category is open, each launch is stamped
// with its own start/end events (launch_k); copies: event pairs recorded on
// the copy stream around each batch of copies.  Sums per category.
enum TimeCat {
  TC_SCORE8, TC_SELECT, TC_SCORE16, TC_CONTROL, TC_COPY, TC_DECODE, TC_DENSE, TC_COMBINE,
  TC_MISC, TC_N
};
struct Timer {
  kvq_ctx *c;
  bool on;
  KernelClock kc{};
  int ncopy = 0;
  int ccat[16];
  Timer(kvq_ctx *ctx, bool timing) : c(ctx), on(timing) {
    kc.ev = c->ev_k;
    kc.cap = 64;
    kc.used = 0;
    kc.open = -1;
    if (on) kernel_clock() = &kc;
  }
  ~Timer() {
    if (on) kernel_clock() = nullptr;
  }
  void open(int k) { kc.open = k; }
  void close() { kc.open = -1; }
  hipError_t copy_begin(int k, hipStream_t st) {
    if (!on || ncopy >= 16) return hipSuccess;
    ccat[ncopy] = k;
    return hipEventRecord(c->ev_c[2 * ncopy], st);
  }
  hipError_t copy_end(hipStream_t st) {
    if (!on || ncopy >= 16) return hipSuccess;
    hipError_t e = hipEventRecord(c->ev_c[2 * ncopy + 1], st);
    ++ncopy;
    return e;
  }
  hipError_t collect(float *ms) {
    for (int k = 0; k < TC_N; ++k) ms[k] = 0.0f;
    for (int u = 0; u < kc.used + ncopy; ++u) {
      const bool kern = u < kc.used;
      hipEvent_t *ev = kern ? c->ev_k + 2 * u : c->ev_c + 2 * (u - kc.used);
      float a = 0.0f;
      hipError_t e = hipEventSynchronize(ev[1]);
      if (e == hipSuccess) e = hipEventElapsedTime(&a, ev[0], ev[1]);
      if (e != hipSuccess) return e;
      ms[kern ? kc.cat[u] : ccat[u - kc.used]] += a;
    }
    return hipSuccess;
  }
};

}  // namespace

extern "C" {

void kvq_default_config(kvq_config *cfg, int32_t n_layers, int32_t max_batch, int32_t n_q_heads,
                        int32_t n_kv_heads, int32_t head_dim, int32_t max_tokens) {
  if (!cfg) return;
  memset(cfg, 0, sizeof(*cfg));
  cfg->n_layers = n_layers;
  cfg->max_batch = max_batch;
  cfg->n_q_heads = n_q_heads;
  cfg->n_kv_heads = n_kv_heads;
  cfg->head_dim = head_dim;
  cfg->max_tokens = max_tokens;
  cfg->tau_cov_ppm = 995000;
  cfg->rho_min_ppm = 900000;
  cfg->widen_rounds = 2;
  cfg->layer_frac_ppm = 500000;
  cfg->eps_key = 1e-3;
  cfg->v_tol = 0.25;
  cfg->flags = 0u;
}

const char *kvq_strerror(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument";
    case KVQ_ENOMEM_DEVICE: return "device allocation failed";
    case KVQ_ENOMEM_HOST: return "pinned host allocation failed";
    case KVQ_ECAPACITY: return "sequence capacity exceeded";
    case KVQ_ESTATE: return "invalid state (empty sequence or bad layer)";
    case KVQ_EHIP: return "HIP runtime error";
    case KVQ_ENOTIMPL: return "not implemented";
    default: return "unknown status";
  }
}

const char *kvq_last_error(const kvq_ctx *ctx) {
  return ctx ? ctx->err.c_str() : noalloc_last_error();
}

double kvq_tier1_bytes_per_token(int32_t d) {
  // K codes d + K meta 4d/64 + V codes d/2 + V meta 4d/32 + eta 4/64
  return (double)d + 4.0 * d / 64.0 + d / 2.0 + 4.0 * d / 32.0 + 4.0 / 64.0;
}

int64_t kvq_device_bytes(const kvq_ctx *ctx) { return ctx ? ctx->dev_bytes : -1; }
int64_t kvq_host_pinned_bytes(const kvq_ctx *ctx) { return ctx ? ctx->host_bytes : -1; }

kvq_status kvq_create(const kvq_config *cfg, kvq_ctx **out) {
  if (!cfg || !out) return KVQ_EINVAL;
  const kvq_config &c = *cfg;
  if (c.n_layers < 1 || c.max_batch < 1 || c.n_q_heads < 1 || c.n_kv_heads < 1 ||
      c.n_kv_heads > 128 ||
      c.n_q_heads % c.n_kv_heads != 0 || (c.head_dim != 64 && c.head_dim != 128) ||
      c.max_tokens < 1 || (c.max_tokens + BLOCK - 1) / BLOCK > MAX_NB)
    return KVQ_EINVAL;
  const int G = c.n_q_heads / c.n_kv_heads;
  if (G != 1 && G != 2 && G != 4) return KVQ_EINVAL;
  const bool kcache = (c.flags & KVQ_FLAG_KEY_CACHE) != 0;
  // cache rows and staging rows are listed as 32-bit row numbers
  if (kcache && ((c.flags & KVQ_FLAG_RESIDENT_KEYS) || c.key_cache_blocks < 1 ||
                 c.key_cache_blocks > ((int64_t)1 << 25) ||
                 (int64_t)c.max_batch * c.n_kv_heads * ((c.max_tokens + BLOCK - 1) / BLOCK) * BLOCK >=
                     ((int64_t)1 << 32)))
    return KVQ_EINVAL;
  if (c.tau_cov_ppm < 1 || c.tau_cov_ppm > 1000000 || c.rho_min_ppm < -1000000 ||
      c.rho_min_ppm > 1000000 || c.widen_rounds < 0 || c.widen_rounds > 12 ||
      c.layer_frac_ppm < 0 || c.layer_frac_ppm > 1000000 || !(c.eps_key >= 0.0) ||
      !(c.v_tol >= 0.0))
    return KVQ_EINVAL;

  kvq_ctx *x = new (std::nothrow) kvq_ctx();
  if (!x) return KVQ_ENOMEM_HOST;
  x->cfg = c;
  (void)hipGetDevice(&x->device);
  Shape &s = x->s;
  s.L = c.n_layers;
  s.Hq = c.n_q_heads;
  s.Hkv = c.n_kv_heads;
  s.G = G;
  s.d = c.head_dim;
  s.NBmax = (c.max_tokens + BLOCK - 1) / BLOCK;
  s.Tmax = s.NBmax * BLOCK;
  s.runmax = s.NBmax / 2 + 1;
  s.nchmax = (s.NBmax + DEC_CB - 1) / DEC_CB;
  s.B = c.max_batch;
  s.kres = (c.flags & KVQ_FLAG_RESIDENT_KEYS) ? 1 : 0;
  s.ncu = 0;
  if (hipDeviceGetAttribute(&s.ncu, hipDeviceAttributeMultiprocessorCount, x->device) !=
          hipSuccess ||
      s.ncu < 1) {
    (void)hipGetLastError();
    delete x;
    return KVQ_EHIP;
  }
  x->th.tau_ppm = c.tau_cov_ppm;
  x->th.rho_ppm = c.rho_min_ppm;
  x->th.R1 = c.widen_rounds;
  x->th.frac_ppm = c.layer_frac_ppm;
  x->th.eps_key = c.eps_key;
  x->th.v_tol = c.v_tol;
  x->th.force_dense = (c.flags & KVQ_FLAG_FORCE_DENSE) ? 1 : 0;
  x->th.fp16_values = (c.flags & KVQ_FLAG_FP16_VALUES) ? 1 : 0;
  x->T.assign((size_t)c.max_batch * c.n_layers, 0);
  x->opar.assign((size_t)c.max_batch * c.n_layers, 0);

  const size_t NU = (size_t)c.max_batch * c.n_layers * c.n_kv_heads;
  const size_t d = s.d, NBm = s.NBmax, Tm = s.Tmax;
  Tier1 &t = x->t;
  Step &w = x->w;
  const size_t B = s.B, Hq = s.Hq, Hkv = s.Hkv;
  hipError_t e = hipSuccess;
#define DA(p, n)                                  \
  if (e == hipSuccess) e = dalloc(x, &(p), (n)); \
  else (void)0
  DA(t.kcodes, NU * NBm * BLOCK * d);
  DA(t.kmeta, NU * NBm * d * 4);
  DA(t.vcodes, NU * NBm * 32 * d);
  DA(t.vmeta, NU * Tm * (d / VGROUP) * 4);
  DA(t.eta, NU * NBm * 4);
  DA(t.vmin, NU * d * 4);
  DA(t.vmax, NU * d * 4);
  DA(t.openk, NU * 2 * BLOCK * d * 2);
  DA(w.qp, B * Hq * d * 4);
  DA(w.shat, B * Hq * Tm * 4);
  DA(w.rlist, B * Hkv * NBm * 4);
  DA(w.sp, B * Hq * Tm * 4);
  DA(w.mhat, B * Hq * NBm * 4);
  DA(w.delta, B * Hq * NBm * 4);
  DA(w.m16, B * Hq * NBm * 4);
  DA(w.Lhat, B * Hq * NBm * 4);
  DA(w.L16, B * Hq * NBm * 4);
  DA(w.What, B * Hq * NBm * 4);
  DA(w.pi, B * Hq * NBm * 4);
  DA(w.Wt, B * Hq * NBm * 4);
  DA(w.W16, B * Hq * NBm * 4);
  DA(w.vh, B * Hq * NBm);
  DA(w.k0, B * Hq * 4);
  DA(w.ssize, B * Hq * 4);
  DA(w.ssd, B * Hq * 8);
  DA(w.ekey64, B * Hq * 8);
  DA(w.eval64, B * Hq * 8);
  DA(w.evs, B * Hq * 2 * 8);
  DA(w.hflags, B * Hq * 4);
  DA(w.hlevel, B * Hq);
  DA(w.U, B * Hkv * NBm);
  DA(w.Knew, B * Hkv * NBm);
  DA(w.V, B * Hkv * NBm);
  DA(w.gstat, B * Hkv * 4);
  DA(w.runs, B * Hkv * 2 * (size_t)s.runmax * 4);
  x->plan_words = 4 + 2 * plan_kcap(s);
  DA(w.plan, x->plan_words * 8);
  DA(w.stage_k, (s.kres ? NU : B * Hkv) * Tm * d * 2);
  t.kres = s.kres ? w.stage_k : nullptr;
  DA(w.stage_v, B * Hkv * Tm * d * 2);
  DA(w.part, B * Hkv * (size_t)s.nchmax * G * (d + 2) * 4);
  DA(w.partd, B * Hkv * (size_t)s.nchmax * G * (d + 2) * 4);
  DA(w.gdense, B * Hkv);
  if (kcache) {
    x->kc.slots = c.key_cache_blocks;
    x->kc.cap = B * Hkv * NBm;
    DA(x->kc.dev, (size_t)c.key_cache_blocks * BLOCK * d * 2);
    DA(x->kc.list_dev, 2 * x->kc.cap * 2 * 4);
  }
#undef DA
  if (e != hipSuccess) {
    x->err = std::string("device allocation: ") + hipGetErrorString(e);
    free_all(x);
    delete x;
    (void)hipGetLastError();
    return KVQ_ENOMEM_DEVICE;
  }
  const size_t t2bytes = NU * Tm * d * 2;
  if (hipHostMalloc((void **)&x->t2k_host, t2bytes, hipHostMallocMapped) != hipSuccess ||
      hipHostMalloc((void **)&x->t2v_host, t2bytes, hipHostMallocMapped) != hipSuccess) {
    free_all(x);
    delete x;
    (void)hipGetLastError();
    return KVQ_ENOMEM_HOST;
  }
  x->host_bytes = (int64_t)(2 * t2bytes);
  void *dk = nullptr, *dv = nullptr;
  e = hipHostGetDevicePointer(&dk, x->t2k_host, 0);
  if (e == hipSuccess) e = hipHostGetDevicePointer(&dv, x->t2v_host, 0);
  x->plan_cap = 4096;
  if (e == hipSuccess) e = hipHostMalloc((void **)&x->plan_host, (4 + x->plan_cap) * 8, 0);
  if (e == hipSuccess) e = hipHostMalloc((void **)&x->u_host, (size_t)c.max_batch * c.n_kv_heads * NBm, 0);
  if (e == hipSuccess)
    e = hipHostMalloc((void **)&x->rlist_host, (size_t)c.max_batch * c.n_kv_heads * NBm * 4, 0);
  x->uppm.assign((size_t)c.n_layers, 0);
  if (e == hipSuccess && kcache) {
    e = hipHostMalloc((void **)&x->kc.list_host, 2 * x->kc.cap * 2 * 4, 0);
    KeyCache &kc = x->kc;
    kc.guard = (int64_t)c.n_layers + 1;
    kc.of.assign(NU * NBm, -1);
    kc.owner.assign((size_t)kc.slots, -1);
    kc.used.assign((size_t)kc.slots, 0);
    kc.prev.assign((size_t)kc.slots, -1);
    kc.next.assign((size_t)kc.slots, -1);
    kc.free_slots.resize((size_t)kc.slots);
    for (int64_t k = 0; k < kc.slots; ++k) kc.free_slots[(size_t)k] = (int32_t)(kc.slots - 1 - k);
  }
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&x->cstream, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&x->ev_start, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&x->ev_copy, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&x->ev_plan, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&x->ev_spec, hipEventDisableTiming);
  for (auto &ev : x->ev_k)
    if (e == hipSuccess) e = hipEventCreate(&ev);
  for (auto &ev : x->ev_c)
    if (e == hipSuccess) e = hipEventCreate(&ev);
  for (auto &ev : x->ev_tot)
    if (e == hipSuccess) e = hipEventCreate(&ev);
  if (e == hipSuccess) e = hipMemsetD32(reinterpret_cast<hipDeviceptr_t>(t.vmin), 0xff800000u, NU * d);
  if (e == hipSuccess) e = hipMemsetD32(reinterpret_cast<hipDeviceptr_t>(t.vmax), 0x007fffffu, NU * d);
  if (e == hipSuccess) e = hipMemset(t.eta, 0, NU * NBm * 4);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    x->err = hipGetErrorString(e);
    free_all(x);
    delete x;
    (void)hipGetLastError();
    return KVQ_EHIP;
  }
  t.t2k = (uint16_t *)dk;
  t.t2v = (uint16_t *)dv;
  *out = x;
  return KVQ_OK;
}

void kvq_destroy(kvq_ctx *ctx) {
  if (!ctx) return;
  free_all(ctx);
  delete ctx;
}

int64_t kvq_seq_len(const kvq_ctx *ctx, int32_t layer, int32_t seq) {
  if (!ctx || layer < 0 || layer >= ctx->cfg.n_layers || seq < 0 || seq >= ctx->cfg.max_batch)
    return KVQ_EINVAL;
  return ctx->T[(size_t)seq * ctx->cfg.n_layers + layer];
}

kvq_status kvq_reset_seq(kvq_ctx *ctx, int32_t seq) {
  if (!ctx || seq < 0 || seq >= ctx->cfg.max_batch) return KVQ_EINVAL;
  const Shape &s = ctx->s;
  // appends to this slot may still run on any stream: their value-range
  // atomics must land before the ranges are cleared
  HIPCK(ctx, hipDeviceSynchronize());
  for (int l = 0; l < s.L; ++l) {
    if (ctx->kc.slots) {
      const int64_t nb = (ctx->T[(size_t)seq * s.L + l] + BLOCK - 1) / BLOCK;
      for (int g = 0; g < s.Hkv; ++g)
        for (int64_t b = 0; b < nb; ++b) ctx->kc.drop((int64_t)unit_of(s, seq, l, g) * s.NBmax + b);
    }
    ctx->T[(size_t)seq * s.L + l] = 0;
    ctx->opar[(size_t)seq * s.L + l] = 0;
    const size_t u0 = unit_of(s, seq, l, 0);
    HIPCK(ctx, hipMemsetD32(reinterpret_cast<hipDeviceptr_t>(ctx->t.vmin + u0 * s.d), 0xff800000u,
                            (size_t)s.Hkv * s.d));
    HIPCK(ctx, hipMemsetD32(reinterpret_cast<hipDeviceptr_t>(ctx->t.vmax + u0 * s.d), 0x007fffffu,
                            (size_t)s.Hkv * s.d));
  }
  HIPCK(ctx, hipDeviceSynchronize());
  return KVQ_OK;
}

kvq_status kvq_append(kvq_ctx *ctx, int32_t layer, int32_t n, const int32_t *seq_ids,
                      const int32_t *n_new, const void *k, const void *v, void *stream) {
  if (!ctx) return KVQ_EINVAL;
  if (layer < 0 || layer >= ctx->cfg.n_layers) return fail(ctx, KVQ_ESTATE, "bad layer");
  if (!valid_seqs(ctx, n, seq_ids) || !n_new) return fail(ctx, KVQ_EINVAL, "bad sequence list");
  const Shape &s = ctx->s;
  AppendArgs a;
  memset(&a, 0, sizeof(a));
  a.n = n;
  a.layer = layer;
  int64_t off = 0;
  int max_blk = 0;
  for (int i = 0; i < n; ++i) {
    if (n_new[i] < 0) return fail(ctx, KVQ_EINVAL, "negative token count");
    const int64_t Told = ctx->T[(size_t)seq_ids[i] * s.L + layer];
    if (Told + n_new[i] > ctx->cfg.max_tokens) return fail(ctx, KVQ_ECAPACITY, "capacity exceeded");
    a.slot[i] = seq_ids[i];
    a.T_old[i] = (int)Told;
    a.n_new[i] = n_new[i];
    a.in_off[i] = (int)off;
    a.par[i] = ctx->opar[(size_t)seq_ids[i] * s.L + layer];
    a.n_blk[i] = n_new[i] > 0 ? (int)((Told + n_new[i] - 1) / BLOCK - Told / BLOCK + 1) : 0;
    max_blk = std::max(max_blk, a.n_blk[i]);
    off += n_new[i];
  }
  if (off > 0 && (!k || !v)) return fail(ctx, KVQ_EINVAL, "null k/v");
  if (off > 0) {
    HIPCK(ctx, launch_append(s, ctx->t, a, (const uint16_t *)k, (const uint16_t *)v, max_blk,
                             (hipStream_t)stream));
  }
  for (int i = 0; i < n; ++i) {
    if (ctx->kc.slots && n_new[i] > 0) {
      // the block holding the old end (if partial) and every new block
      const int64_t b0 = a.T_old[i] / BLOCK, b1 = (a.T_old[i] + n_new[i] - 1) / BLOCK;
      for (int g = 0; g < s.Hkv; ++g)
        for (int64_t b = b0; b <= b1; ++b)
          ctx->kc.drop((int64_t)unit_of(s, seq_ids[i], layer, g) * s.NBmax + b);
    }
    ctx->T[(size_t)seq_ids[i] * s.L + layer] += n_new[i];
    if (n_new[i] > 0) ctx->opar[(size_t)seq_ids[i] * s.L + layer] ^= 1;
  }
  return KVQ_OK;
}

namespace {

struct Plan {
  int64_t nk = 0, nv = 0;
  uint32_t flags = 0;
  bool flagged = false;   // the first controller round flagged a head
  std::vector<unsigned long long> ent;
};

// The plan's header and first entries come back in one copy on the step's
// stream; the host waits for that copy only (an event), so kernels enqueued
// after it keep running meanwhile.
kvq_status read_plan_issue(kvq_ctx *c, hipStream_t st) {
  const size_t first = std::min(c->plan_cap, plan_kcap(c->s));
  HIPCK(c, hipMemcpyAsync(c->plan_host, c->w.plan, (4 + first) * 8, hipMemcpyDeviceToHost, st));
  HIPCK(c, hipEventRecord(c->ev_plan, st));
  return KVQ_OK;
}

kvq_status read_plan_wait(kvq_ctx *c, Plan &p) {
  const size_t kcap = plan_kcap(c->s);
  const size_t first = std::min(c->plan_cap, kcap);
  HIPCK(c, hipEventSynchronize(c->ev_plan));
  p.nk = (int64_t)c->plan_host[0];
  p.nv = (int64_t)c->plan_host[1];
  p.flags = (uint32_t)c->plan_host[2];
  p.flagged = c->plan_host[3] != 0ull;
  if (p.nk < 0 || (size_t)p.nk > kcap || p.nv < 0 || (size_t)p.nv > kcap)
    return fail(c, KVQ_EHIP, "promotion plan out of range");
  p.ent.assign(c->plan_host + 4, c->plan_host + 4 + std::min((size_t)p.nk, first));
  if ((size_t)p.nk > first) {
    p.ent.resize((size_t)p.nk);
    HIPCK(c, hipMemcpy(p.ent.data() + first, c->w.plan + 4 + first, ((size_t)p.nk - first) * 8,
                       hipMemcpyDeviceToHost));
  }
  if (p.nv > 0) {
    const size_t k0 = p.ent.size();
    p.ent.resize(k0 + (size_t)p.nv);
    HIPCK(c, hipMemcpy(p.ent.data() + k0, c->w.plan + 4 + kcap, (size_t)p.nv * 8,
                       hipMemcpyDeviceToHost));
  }
  return KVQ_OK;
}

kvq_status read_plan(kvq_ctx *c, hipStream_t st, Plan &p) {
  const kvq_status r = read_plan_issue(c, st);
  return r != KVQ_OK ? r : read_plan_wait(c, p);
}

// After the selection: the group unions U of the call's sequences come back
// (one copy on the step's stream), and the plan's key entries are their runs
// of consecutive blocks, one entry per run (the layout of the device plan).
kvq_status read_union(kvq_ctx *c, hipStream_t st, const SeqTab &tab, Plan &p, int64_t &ublocks) {
  const Shape &s = c->s;
  const size_t rows = (size_t)tab.n * s.Hkv;
  HIPCK(c, hipMemcpyAsync(c->u_host, c->w.U, rows * s.NBmax, hipMemcpyDeviceToHost, st));
  HIPCK(c, hipEventRecord(c->ev_plan, st));
  HIPCK(c, hipEventSynchronize(c->ev_plan));
  p = Plan();
  for (int i = 0; i < tab.n; ++i) {
    const int NB = tab.nbc[i + 1] - tab.nbc[i];
    for (int g = 0; g < s.Hkv; ++g) {
      const size_t ig = (size_t)i * s.Hkv + g;
      const uint8_t *u = c->u_host + ig * s.NBmax;
      int b = 0;
      while (b < NB) {
        // eight flags at a time while they are all clear or all set
        if (b + 8 <= NB) {
          uint64_t x;
          memcpy(&x, u + b, 8);
          if (x == 0ull) {
            b += 8;
            continue;
          }
        }
        if (!u[b]) {
          ++b;
          continue;
        }
        int e = b + 1;
        while (e + 8 <= NB) {
          uint64_t x;
          memcpy(&x, u + e, 8);
          if (x != 0x0101010101010101ull) break;
          e += 8;
        }
        while (e < NB && u[e]) ++e;
        p.ent.push_back((unsigned long long)(e - b) | ((unsigned long long)b << 16) |
                        ((unsigned long long)ig << 32));
        b = e;
      }
    }
  }
  p.nk = (int64_t)p.ent.size();
  ublocks = 0;
  for (const unsigned long long e : p.ent) ublocks += (int64_t)(e & 0xffffu);
  return KVQ_OK;
}

// U fraction (ppm) of a layer's last step from which the next step defers
// the INT8 scores (kvq_selftest_defer_scores changes it).
constexpr int32_t DEFER_PPM = 750000;
static int32_t g_defer_ppm = DEFER_PPM;
static_assert((int64_t)MAX_CALL * 128 <= 65536 && MAX_NB <= 65536, "rescore entries are ig << 16 | block");

// The call's units outside U (ig << 16 | block), from the unions read back.
int outside_union(kvq_ctx *c, const SeqTab &tab) {
  const Shape &s = c->s;
  int n = 0;
  for (int i = 0; i < tab.n; ++i) {
    const int NB = tab.nbc[i + 1] - tab.nbc[i];
    for (int g = 0; g < s.Hkv; ++g) {
      const size_t ig = (size_t)i * s.Hkv + g;
      const uint8_t *u = c->u_host + ig * s.NBmax;
      for (int b = 0; b < NB; ++b) {
        if (b + 8 <= NB && (b & 7) == 0) {
          uint64_t x;
          memcpy(&x, u + b, 8);
          if (x == 0x0101010101010101ull) {
            b += 7;
            continue;
          }
        }
        if (!u[b]) c->rlist_host[n++] = (uint32_t)(ig << 16) | (uint32_t)b;
      }
    }
  }
  return n;
}

// Issues the copies of a plan on the copy stream; returns bytes and blocks.
// With the key cache, a key run splits into cached blocks (one device-side
// gather from their slots) and runs of uncached blocks (host link), and the
// uncached blocks that find a slot are copied into it from the staging
// buffer once their host copies have landed.
// Plan entries with overlapping or adjacent runs of one (sequence, KV head)
// and kind merged (the selection lists each query head's runs; later rounds
// list each group's new blocks once), in (kind, group, start) order.
void merge_runs(const std::vector<unsigned long long> &ent, std::vector<unsigned long long> &out) {
  // an entry (len | start << 16 | ig << 32 | kind << 48) sorts by kind,
  // group, start
  std::vector<unsigned long long> v(ent);
  std::sort(v.begin(), v.end());
  out.clear();
  out.reserve(v.size());
  for (const unsigned long long e : v) {
    const unsigned long long grp = e >> 32;
    const unsigned long long st = (e >> 16) & 0xffffu, en = st + (e & 0xffffu);
    if (!out.empty() && (out.back() >> 32) == grp) {
      const unsigned long long pst = (out.back() >> 16) & 0xffffu;
      const unsigned long long pen = pst + (out.back() & 0xffffu);
      if (st <= pen) {
        const unsigned long long nen = std::max(pen, en);
        out.back() = (grp << 32) | (pst << 16) | (nen - pst);
        continue;
      }
    }
    out.push_back(e);
  }
}

kvq_status issue_copies(kvq_ctx *c, const SeqTab &tab, int layer, const Plan &p, int64_t &bytes,
                        int64_t &kblocks, int64_t &vblocks, int64_t &kcached) {
  const Shape &s = c->s;
  const size_t blk_bytes = (size_t)BLOCK * s.d * 2;
  KeyCache &kc = c->kc;
  uint32_t *hits = kc.list_host, *adm = kc.list_host ? kc.list_host + 2 * kc.cap : nullptr;
  size_t nh = 0, na = 0;
  auto h2d = [&](int kind, size_t u, int ig, int start, int len) -> kvq_status {
    const size_t srow = u * s.Tmax + (size_t)start * BLOCK;
    const size_t drow = (size_t)ig * s.Tmax + (size_t)start * BLOCK;
    uint16_t *dst = (kind ? c->w.stage_v : c->w.stage_k) + drow * s.d;
    const uint16_t *src = (kind ? c->t2v_host : c->t2k_host) + srow * s.d;
    HIPCK(c, hipMemcpyAsync(dst, src, (size_t)len * blk_bytes, hipMemcpyHostToDevice, c->cstream));
    bytes += (int64_t)len * (int64_t)blk_bytes;
    (kind ? vblocks : kblocks) += len;
    return KVQ_OK;
  };
  std::vector<unsigned long long> runs;
  merge_runs(p.ent, runs);
  for (const unsigned long long e : runs) {
    const int len = (int)(e & 0xffffu), start = (int)((e >> 16) & 0xffffu);
    const int ig = (int)((e >> 32) & 0xffffu), kind = (int)((e >> 48) & 1u);
    const int i = ig / s.Hkv, g = ig % s.Hkv;
    const size_t u = unit_of(s, tab.slot[i], layer, g);
    if (kind == 0 && s.kres) {   // resident keys: already in device memory
      kblocks += len;
      continue;
    }
    if (kind == 1 || !kc.slots) {
      const kvq_status r = h2d(kind, u, ig, start, len);
      if (r != KVQ_OK) return r;
      continue;
    }
    if (start + len > s.NBmax || (size_t)ig >= (size_t)s.B * s.Hkv)
      return fail(c, KVQ_EHIP, "promotion entry out of range");
    const int64_t key0 = (int64_t)u * s.NBmax;
    const uint32_t row0 = (uint32_t)((size_t)ig * s.Tmax);
    for (int b = start; b < start + len;) {
      const int32_t x = kc.of[(size_t)(key0 + b)];
      if (x >= 0) {                     // cached: gather from the slot
        kc.touch(x);
        hits[2 * nh] = (uint32_t)x * BLOCK;
        hits[2 * nh + 1] = row0 + (uint32_t)b * BLOCK;
        ++nh;
        ++kcached;
        ++b;
        continue;
      }
      int e2 = b + 1;
      while (e2 < start + len && kc.of[(size_t)(key0 + e2)] < 0) ++e2;
      const kvq_status r = h2d(0, u, ig, b, e2 - b);
      if (r != KVQ_OK) return r;
      for (int bb = b; bb < e2; ++bb) {
        const int32_t y = kc.admit(key0 + bb);
        if (y < 0) break;               // every slot protected: no further admission
        adm[2 * na] = row0 + (uint32_t)bb * BLOCK;
        adm[2 * na + 1] = (uint32_t)y * BLOCK;
        ++na;
      }
      b = e2;
    }
  }
  if (nh > kc.cap || na > kc.cap) return fail(c, KVQ_EHIP, "cache list overflow");
  // the gather (slots -> staging), then the admissions (staging -> slots,
  // after the host copies on this stream); each list goes over first
  if (nh > 0) {
    HIPCK(c, hipMemcpyAsync(kc.list_dev, hits, nh * 8, hipMemcpyHostToDevice, c->cstream));
    HIPCK(c, launch_copy_blocks(kc.list_dev, (int)nh, kc.dev, c->w.stage_k, s.d, c->cstream));
  }
  if (na > 0) {
    HIPCK(c, hipMemcpyAsync(kc.list_dev + 2 * kc.cap, adm, na * 8, hipMemcpyHostToDevice,
                            c->cstream));
    HIPCK(c, launch_copy_blocks(kc.list_dev + 2 * kc.cap, (int)na, c->w.stage_k, kc.dev, s.d,
                                c->cstream));
  }
  return KVQ_OK;
}

}  // namespace

kvq_status kvq_decode_step(kvq_ctx *ctx, int32_t layer, int32_t n, const int32_t *seq_ids,
                           const void *q, float *out, float *e_key, float *e_val, int8_t *level,
                           kvq_step_stats *stats, void *stream) {
  if (!ctx) return KVQ_EINVAL;
  if (layer < 0 || layer >= ctx->cfg.n_layers) return fail(ctx, KVQ_ESTATE, "bad layer");
  if (!valid_seqs(ctx, n, seq_ids)) return fail(ctx, KVQ_EINVAL, "bad sequence list");
  if (!q || !out || !e_key || !e_val || !level) return fail(ctx, KVQ_EINVAL, "null output");
  const Shape &s = ctx->s;
  SeqTab tab;
  memset(&tab, 0, sizeof(tab));
  tab.n = n;
  int maxNB = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t T = ctx->T[(size_t)seq_ids[i] * s.L + layer];
    if (T < 1) return fail(ctx, KVQ_ESTATE, "decode on an empty sequence");
    tab.slot[i] = seq_ids[i];
    tab.T[i] = (int)T;
    tab.nbc[i + 1] = tab.nbc[i] + (int)((T + BLOCK - 1) / BLOCK);
    maxNB = std::max(maxNB, (int)((T + BLOCK - 1) / BLOCK));
  }
  hipStream_t st = (hipStream_t)stream;
  // kernel and copy events only when the call returns statistics: a launch
  // with start/stop events costs several microseconds of dispatch gap
  const bool timing = stats && (ctx->cfg.flags & KVQ_FLAG_TIMING) != 0;
  Step &w = ctx->w;
  const size_t NBm = s.NBmax;
  int64_t h2d = 0, kblk = 0, vblk = 0, dense_heads = 0, kcached = 0;
  ++ctx->kc.now;
  int syncs = 0, rounds = 0;
  bool decoded = false;   // the decode launched behind the last round stands
  bool spec = false;      // a speculative decode was enqueued (ev_spec recorded)
  Timer tm{ctx, timing};
  if (timing) HIPCK(ctx, hipEventRecord(ctx->ev_tot[0], st));

  const float C = (float)(1.4426950408889634 / sqrt((double)s.d));
  // staging may still be read by the previous step's kernels, and tier 2 was
  // written by earlier appends on this stream: copies wait for both
  HIPCK(ctx, hipEventRecord(ctx->ev_start, st));
  HIPCK(ctx, hipStreamWaitEvent(ctx->cstream, ctx->ev_start, 0));

  // with resident keys no copy depends on the selection, so the host reads
  // the unions only for the statistics
  const bool read_u = !s.kres || stats;
  // The INT8 scores ŝ′ are read later only for blocks outside U.  When the
  // last step at this layer put at least three quarters of the blocks in U,
  // the pass stores none and the blocks outside U are rescored after the
  // selection (a written byte costs about four read bytes here); otherwise,
  // or when the unions are not read back, the pass stores them all.
  const bool defer = read_u && !(ctx->cfg.flags & KVQ_FLAG_ALL_SCORES) &&
                     ctx->uppm[(size_t)layer] >= g_defer_ppm;
  tm.open(TC_SCORE8);   // INT8 scores, with the step set-up (q', flags cleared)
  HIPCK(ctx, launch_score_int8(s, ctx->t, w, tab, layer, (const uint16_t *)q, C, !defer, st));
  tm.open(TC_SELECT);
  HIPCK(ctx, launch_select(s, w, tab, ctx->th.tau_ppm, maxNB, st));
  tm.close();
  Plan plan;
  kvq_status rs = KVQ_OK;
  int nres = 0;   // blocks outside U whose ŝ′ the first controller round computes
  bool fused_resc = false;   // ... or the fused first round's decode waves, each for its own
  if (read_u) {
    int64_t ublocks = 0;
    rs = read_union(ctx, st, tab, plan, ublocks);
    if (rs != KVQ_OK) return rs;
    ++syncs;
    const int64_t all = (int64_t)tab.nbc[n] * s.Hkv;
    ctx->uppm[(size_t)layer] = all > 0 ? (int32_t)(ublocks * 1000000 / all) : 0;
    if (defer) {
      nres = outside_union(ctx, tab);
      // Who computes them: in a first round fused with the decode (the one
      // kernel that reads them), each decode wave for its own blocks; in a
      // first round with a launch of its own, extra workgroups beside the
      // heads' evaluation (from the list); in a step that starts with the
      // group pass (FP16 values, forced dense), a launch of their own, here
      const bool ctl = !ctx->th.force_dense && !ctx->th.fp16_values;
      fused_resc = nres > 0 && ctl && eval_decode_fits(s, tab);
      if (fused_resc) {
        nres = 0;
      } else if (nres > 0) {
        HIPCK(ctx, hipMemcpyAsync(w.rlist, ctx->rlist_host, (size_t)nres * 4, hipMemcpyHostToDevice, st));
        if (!ctl) {
          tm.open(TC_SCORE8);
          HIPCK(ctx, launch_rescore_int8(s, ctx->t, w, tab, layer, (const uint16_t *)q, C, w.rlist, nres, st));
          tm.close();
          nres = 0;
        }
      }
    }
  } else {
    plan.nk = 1;   // score whatever the selection flagged
  }
  for (int round = 0;; ++round) {
    const bool new_keys = plan.nk > 0;
    if (!plan.ent.empty()) {
      if (spec) HIPCK(ctx, hipStreamWaitEvent(ctx->cstream, ctx->ev_spec, 0));
      HIPCK(ctx, tm.copy_begin(TC_COPY, ctx->cstream));
      rs = issue_copies(ctx, tab, layer, plan, h2d, kblk, vblk, kcached);
      if (rs != KVQ_OK) return rs;
      HIPCK(ctx, tm.copy_end(ctx->cstream));
      HIPCK(ctx, hipEventRecord(ctx->ev_copy, ctx->cstream));
      HIPCK(ctx, hipStreamWaitEvent(st, ctx->ev_copy, 0));
    }
    if (round > 0 && !(plan.flags & 1u)) break;      // every group final
    if (round > ctx->th.R1) return fail(ctx, KVQ_EHIP, "controller did not finish its rounds");
    if (new_keys) {
      tm.open(TC_SCORE16);
      HIPCK(ctx, launch_score_fp16(s, w, tab, layer, maxNB, st));
    }
    // The first round evaluates every head (k_eval) and flags the heads the
    // group decisions would act on (ranking failure, E_key > eps_key, E_val
    // > v_tol).  In the common case none is flagged: every level is 0 and the
    // speculative combine below writes the outputs, so the group pass
    // (k_decide) does not run.  Otherwise k_decide runs for this round and
    // the rounds go on as below.
    const bool first = round == 0 && !ctx->th.force_dense && !ctx->th.fp16_values;
    // The first round's evaluation and the speculative decode (which reads
    // only U, the scores and the block maxima) share one launch, the decode's
    // chunks filling the compute units the heads leave idle; fused_extra is
    // that launch's count of workgroups beside the decode's (for the
    // combine), or -1 when they run as separate launches.
    int fused_extra = -1;
    if (first) {
      tm.open(TC_DECODE);
      HIPCK(ctx, launch_eval_decode(s, ctx->t, w, tab, layer, ctx->th, maxNB, (const uint16_t *)q, C,
                                    fused_resc, &fused_extra, st));
      if (fused_resc && fused_extra < 0) return fail(ctx, KVQ_EHIP, "fused first round not launched");
      if (fused_extra < 0) {
        tm.open(TC_CONTROL);
        HIPCK(ctx, launch_eval(s, ctx->t, w, tab, layer, ctx->th, maxNB, (const uint16_t *)q, C, w.rlist,
                               nres, st));
      }
    } else {
      tm.open(TC_CONTROL);
      HIPCK(ctx, launch_control(s, ctx->t, w, tab, layer, ctx->th, round, maxNB, st));
    }
    rs = read_plan_issue(ctx, st);
    if (rs != KVQ_OK) return rs;
    // the decode and combine go in behind the plan's copy: in the common case
    // (no group widens, no values to copy, no head at rung 3) they are the
    // step's last kernels and run while the host reads the plan; otherwise
    // they are launched again below and overwrite these results.  They read
    // the value staging of blocks this round may have flagged for rung 2,
    // whose copies are issued only after the plan is read: every later copy
    // waits for them (ev_spec), so no copy writes a buffer they still read.
    if (!ctx->th.force_dense) {
      if (fused_extra < 0) {
        tm.open(TC_DECODE);
        // (the first round only evaluates: no value is promoted yet)
        HIPCK(ctx, launch_decode(s, ctx->t, w, tab, layer, !first, st));
      }
      tm.open(TC_COMBINE);
      // mixed partials for every head: the result is kept only if no head
      // reached rung 3
      HIPCK(ctx, launch_combine(s, w, tab, out, first ? 3 : 1, e_key, e_val, level, fused_extra, st));
      HIPCK(ctx, hipEventRecord(ctx->ev_spec, st));
      spec = true;
    }
    tm.close();
    rs = read_plan_wait(ctx, plan);
    if (rs != KVQ_OK) return rs;
    ++syncs;
    rounds = round + 1;
    if (first && !plan.flagged) {
      decoded = true;
      break;
    }
    if (first) {
      // a flagged head: the group decisions of this round, and a new plan
      tm.open(TC_CONTROL);
      HIPCK(ctx, launch_decide(s, ctx->t, w, tab, layer, ctx->th, round, maxNB, st));
      tm.close();
      rs = read_plan(ctx, st, plan);
      if (rs != KVQ_OK) return rs;
      ++syncs;
    }
    if (!(plan.flags & 1u) && plan.ent.empty()) {
      // outputs of the speculative combine stand unless a head is at rung 3;
      // after a flagged first round they came from the first round's sums
      decoded = !first && !ctx->th.force_dense && !(plan.flags & 2u);
      break;
    }
  }
  // rung 4 and the outputs: with no head at rung 3 (and no forced dense
  // fallback) no level can change, and the combine kernel writes the outputs
  const bool maybe_dense = ctx->th.force_dense || (plan.flags & 2u);
  if (!decoded) {
    if (maybe_dense) {
      tm.open(TC_MISC);
      HIPCK(ctx, launch_finalize(s, w, tab, ctx->th, e_key, e_val, level, st));
      tm.close();
    }
    std::vector<uint8_t> gd;
    if (maybe_dense) {
      gd.resize((size_t)n * s.Hkv);
      HIPCK(ctx, hipMemcpyAsync(gd.data(), w.gdense, gd.size(), hipMemcpyDeviceToHost, st));
      HIPCK(ctx, hipStreamSynchronize(st));
      ++syncs;
      bool any = false;
      if (spec) HIPCK(ctx, hipStreamWaitEvent(ctx->cstream, ctx->ev_spec, 0));
      for (int i = 0; i < n; ++i)
        for (int g = 0; g < s.Hkv; ++g) {
          if (!gd[(size_t)i * s.Hkv + g]) continue;
          any = true;
          ++dense_heads;
          const size_t u = unit_of(s, tab.slot[i], layer, g);
          const size_t ig = (size_t)i * s.Hkv + g;
          const size_t bytes = (size_t)((tab.T[i] + BLOCK - 1) / BLOCK) * BLOCK * s.d * 2;
          HIPCK(ctx, tm.copy_begin(TC_COPY, ctx->cstream));
          if (!s.kres) {   // resident keys are in device memory already
            HIPCK(ctx, hipMemcpyAsync(w.stage_k + ig * s.Tmax * s.d, ctx->t2k_host + u * s.Tmax * s.d,
                                      bytes, hipMemcpyHostToDevice, ctx->cstream));
            h2d += (int64_t)bytes;
          }
          HIPCK(ctx, hipMemcpyAsync(w.stage_v + ig * s.Tmax * s.d, ctx->t2v_host + u * s.Tmax * s.d,
                                    bytes, hipMemcpyHostToDevice, ctx->cstream));
          HIPCK(ctx, tm.copy_end(ctx->cstream));
          h2d += (int64_t)bytes;
        }
      if (any) {
        HIPCK(ctx, hipEventRecord(ctx->ev_copy, ctx->cstream));
        HIPCK(ctx, hipStreamWaitEvent(st, ctx->ev_copy, 0));
        tm.open(TC_DENSE);
        HIPCK(ctx, launch_dense_staged(s, w, tab, layer, (const uint16_t *)q, maxNB, st));
        tm.close();
      }
    }
    if (!ctx->th.force_dense) {        // forced: every head is at level 4 (dense partials)
      tm.open(TC_DECODE);
      HIPCK(ctx, launch_decode(s, ctx->t, w, tab, layer, true, st));
    }
    tm.open(TC_COMBINE);
    HIPCK(ctx, launch_combine(s, w, tab, out, 0, maybe_dense ? nullptr : e_key,
                              maybe_dense ? nullptr : e_val, maybe_dense ? nullptr : level, -1, st));
    tm.close();
  }
  if (timing) HIPCK(ctx, hipEventRecord(ctx->ev_tot[1], st));

  ctx->last_n = n;
  ctx->last_layer = layer;
  for (int i = 0; i < n; ++i) {
    ctx->last_slot[i] = tab.slot[i];
    ctx->last_T[i] = tab.T[i];
  }
  if (stats) {
    memset(stats, 0, sizeof(*stats));
    stats->promoted_key_blocks = kblk;
    stats->cached_key_blocks = kcached;
    stats->scores_deferred = defer ? 1 : 0;
    stats->promoted_value_blocks = vblk;
    stats->dense_kv_heads = dense_heads;
    stats->h2d_bytes = h2d;
    stats->key_rounds = rounds;
    stats->host_syncs = syncs;
    std::vector<int8_t> lv((size_t)n * s.Hq);
    HIPCK(ctx, hipMemcpyAsync(lv.data(), level, lv.size(), hipMemcpyDeviceToHost, st));
    HIPCK(ctx, hipStreamSynchronize(st));
    for (int8_t x : lv)
      if (x >= 0 && x <= 4) stats->level_count[(int)x]++;
    if (timing) {
      float ms[TC_N];
      HIPCK(ctx, tm.collect(ms));
      stats->ms_score_int8 = ms[TC_SCORE8];
      stats->ms_select = ms[TC_SELECT];
      stats->ms_score_fp16 = ms[TC_SCORE16];
      stats->ms_control = ms[TC_CONTROL];
      stats->ms_copy = ms[TC_COPY];
      stats->ms_decode = ms[TC_DECODE];
      stats->ms_dense = ms[TC_DENSE];
      stats->ms_combine = ms[TC_COMBINE];
      stats->ms_misc = ms[TC_MISC];
      float a = 0.0f;
      HIPCK(ctx, hipEventSynchronize(ctx->ev_tot[1]));
      HIPCK(ctx, hipEventElapsedTime(&a, ctx->ev_tot[0], ctx->ev_tot[1]));
      stats->ms_total = a;
    }
  }
  return KVQ_OK;
}

// ---- comparators ------------------------------------------------------------------

kvq_status kvq_decode_naive(kvq_ctx *ctx, int32_t layer, int32_t n, const int32_t *seq_ids,
                            const void *q, float *out, void *stream) {
  if (!ctx) return KVQ_EINVAL;
  if (layer < 0 || layer >= ctx->cfg.n_layers) return fail(ctx, KVQ_ESTATE, "bad layer");
  if (!valid_seqs(ctx, n, seq_ids)) return fail(ctx, KVQ_EINVAL, "bad sequence list");
  if (!q || !out) return fail(ctx, KVQ_EINVAL, "null argument");
  const Shape &s = ctx->s;
  SeqTab tab;
  memset(&tab, 0, sizeof(tab));
  tab.n = n;
  int maxNB = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t T = ctx->T[(size_t)seq_ids[i] * s.L + layer];
    if (T < 1) return fail(ctx, KVQ_ESTATE, "decode on an empty sequence");
    tab.slot[i] = seq_ids[i];
    tab.T[i] = (int)T;
    tab.nbc[i + 1] = tab.nbc[i] + (int)((T + BLOCK - 1) / BLOCK);
    maxNB = std::max(maxNB, (int)((T + BLOCK - 1) / BLOCK));
  }
  hipStream_t st = (hipStream_t)stream;
  Step &w = ctx->w;
  // empty U and V: INT8 scores and INT4 values for every block
  const float C = (float)(1.4426950408889634 / sqrt((double)s.d));
  HIPCK(ctx, launch_score_int8(s, ctx->t, w, tab, layer, (const uint16_t *)q, C, true, st));
  HIPCK(ctx, launch_decode(s, ctx->t, w, tab, layer, false, st));
  HIPCK(ctx, launch_combine(s, w, tab, out, 1, nullptr, nullptr, nullptr, -1, st));
  return KVQ_OK;
}

kvq_status kvq_dense_decode(kvq_ctx *ctx, int32_t n, const int32_t *seq_lens, const void *q,
                            const void *k, const void *v, float *out, void *stream) {
  if (!ctx) return KVQ_EINVAL;
  if (n < 1 || n > ctx->cfg.max_batch || n > MAX_CALL || !seq_lens)
    return fail(ctx, KVQ_EINVAL, "bad sequence count");
  if (!q || !k || !v || !out) return fail(ctx, KVQ_EINVAL, "null argument");
  const Shape &s = ctx->s;
  DenseArgs a;
  memset(&a, 0, sizeof(a));
  SeqTab tab;
  memset(&tab, 0, sizeof(tab));
  a.n = tab.n = n;
  int maxNB = 0;
  for (int i = 0; i < n; ++i) {
    if (seq_lens[i] < 1 || seq_lens[i] > ctx->cfg.max_tokens)
      return fail(ctx, KVQ_EINVAL, "sequence length out of range");
    a.T[i] = tab.T[i] = seq_lens[i];
    tab.nbc[i + 1] = tab.nbc[i] + (seq_lens[i] + BLOCK - 1) / BLOCK;
    maxNB = std::max(maxNB, (seq_lens[i] + BLOCK - 1) / BLOCK);
  }
  a.tcap = ctx->cfg.max_tokens;
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.v = (const uint16_t *)v;
  hipStream_t st = (hipStream_t)stream;
  HIPCK(ctx, launch_dense_vram(s, ctx->w, a, maxNB, st));
  HIPCK(ctx, launch_combine(s, ctx->w, tab, out, 2, nullptr, nullptr, nullptr, -1, st));
  return KVQ_OK;
}

// ---- test and debug exports -----------------------------------------------------

int64_t kvq_tier1_export_bytes(const kvq_ctx *ctx, int32_t layer, int32_t seq) {
  if (!ctx || layer < 0 || layer >= ctx->cfg.n_layers || seq < 0 || seq >= ctx->cfg.max_batch)
    return KVQ_EINVAL;
  const int64_t T = ctx->T[(size_t)seq * ctx->cfg.n_layers + layer];
  const int64_t NB = (T + BLOCK - 1) / BLOCK, d = ctx->s.d;
  return T * d + NB * d * 2 * 2 + NB * 4 + T * d + T * (d / 32) * 2 * 2 + d * 4 * 2;
}

kvq_status kvq_export_tier1(kvq_ctx *ctx, int32_t layer, int32_t seq, int32_t g, void *host_dst,
                            size_t bytes) {
  if (!ctx || !host_dst) return KVQ_EINVAL;
  const int64_t need = kvq_tier1_export_bytes(ctx, layer, seq);
  if (need < 0 || (size_t)need != bytes || g < 0 || g >= ctx->s.Hkv)
    return fail(ctx, KVQ_EINVAL, "bad export request");
  const Shape &s = ctx->s;
  const int T = (int)ctx->T[(size_t)seq * s.L + layer];
  const int NB = (T + BLOCK - 1) / BLOCK, d = s.d;
  const size_t u = unit_of(s, seq, layer, g);
  HIPCK(ctx, hipDeviceSynchronize());
  uint8_t *p = (uint8_t *)host_dst;
  if (T > 0) {
    uint8_t *tmp = nullptr;
    HIPCK(ctx, hipMalloc(&tmp, (size_t)T * d));
    hipError_t e = launch_export_kcodes(s, ctx->t, u, T, tmp, nullptr);
    if (e == hipSuccess) e = hipMemcpy(p, tmp, (size_t)T * d, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = launch_export_vcodes(s, ctx->t, u, T, tmp, nullptr);
    if (e == hipSuccess)
      e = hipMemcpy(p + (size_t)T * d + (size_t)NB * d * 4 + (size_t)NB * 4, tmp, (size_t)T * d,
                    hipMemcpyDeviceToHost);
    (void)hipFree(tmp);
    HIPCK(ctx, e);
  }
  std::vector<uint32_t> km((size_t)NB * d), vm((size_t)T * (d / 32)), mn(d), mx(d);
  HIPCK(ctx, hipMemcpy(km.data(), ctx->t.kmeta + u * s.NBmax * d, km.size() * 4, hipMemcpyDeviceToHost));
  HIPCK(ctx, hipMemcpy(vm.data(), ctx->t.vmeta + u * s.Tmax * (d / 32), vm.size() * 4,
                       hipMemcpyDeviceToHost));
  HIPCK(ctx, hipMemcpy(mn.data(), ctx->t.vmin + u * d, (size_t)d * 4, hipMemcpyDeviceToHost));
  HIPCK(ctx, hipMemcpy(mx.data(), ctx->t.vmax + u * d, (size_t)d * 4, hipMemcpyDeviceToHost));
  uint8_t *q = p + (size_t)T * d;
  uint16_t *ks = (uint16_t *)q, *ko = ks + (size_t)NB * d;
  for (size_t k = 0; k < km.size(); ++k) {
    ks[k] = (uint16_t)(km[k] & 0xffffu);
    ko[k] = (uint16_t)(km[k] >> 16);
  }
  q += (size_t)NB * d * 4;
  HIPCK(ctx, hipMemcpy(q, ctx->t.eta + u * s.NBmax, (size_t)NB * 4, hipMemcpyDeviceToHost));
  q += (size_t)NB * 4 + (size_t)T * d;
  uint16_t *vs = (uint16_t *)q, *vo = vs + vm.size();
  for (size_t k = 0; k < vm.size(); ++k) {
    vs[k] = (uint16_t)(vm[k] & 0xffffu);
    vo[k] = (uint16_t)(vm[k] >> 16);
  }
  q += vm.size() * 4;
  float *fmn = (float *)q, *fmx = fmn + d;
  auto unord = [](uint32_t x) {
    uint32_t b = (x & 0x80000000u) ? (x & 0x7fffffffu) : ~x;
    float f;
    memcpy(&f, &b, 4);
    return f;
  };
  for (int c = 0; c < d; ++c) {
    fmn[c] = unord(mn[c]);
    fmx[c] = unord(mx[c]);
  }
  return KVQ_OK;
}

int64_t kvq_trace_bytes(const kvq_ctx *ctx, int32_t which, int32_t seq) {
  if (!ctx) return KVQ_EINVAL;
  int i = -1;
  for (int k = 0; k < ctx->last_n; ++k)
    if (ctx->last_slot[k] == seq) i = k;
  if (i < 0) return KVQ_ESTATE;
  const int64_t T = ctx->last_T[i], NB = (T + BLOCK - 1) / BLOCK;
  const int64_t Hq = ctx->s.Hq, Hkv = ctx->s.Hkv;
  switch (which) {
    case KVQ_TR_SHAT: case KVQ_TR_SP: return Hq * T * 4;
    case KVQ_TR_MHAT: case KVQ_TR_LHAT: case KVQ_TR_DELTA: case KVQ_TR_M16: case KVQ_TR_L16:
    case KVQ_TR_WHAT: case KVQ_TR_PI: case KVQ_TR_WT: case KVQ_TR_W16: return Hq * NB * 4;
    case KVQ_TR_K0: case KVQ_TR_SSIZE: case KVQ_TR_HFLAGS: return Hq * 4;
    case KVQ_TR_SSD: case KVQ_TR_EKEY64: case KVQ_TR_EVAL64: return Hq * 8;
    case KVQ_TR_U: case KVQ_TR_V: return Hkv * NB;
    case KVQ_TR_VH: return Hq * NB;
    default: return KVQ_EINVAL;
  }
}

kvq_status kvq_export_trace(kvq_ctx *ctx, int32_t which, int32_t seq, void *host_dst, size_t bytes) {
  const int64_t need = kvq_trace_bytes(ctx, which, seq);
  if (need < 0) return (kvq_status)need;
  if (!host_dst || (size_t)need != bytes) return fail(ctx, KVQ_EINVAL, "bad trace request");
  int i = 0;
  for (int k = 0; k < ctx->last_n; ++k)
    if (ctx->last_slot[k] == seq) i = k;
  const Shape &s = ctx->s;
  const Step &w = ctx->w;
  const int64_t T = ctx->last_T[i], NB = (T + BLOCK - 1) / BLOCK;
  HIPCK(ctx, hipDeviceSynchronize());
  uint8_t *dst = (uint8_t *)host_dst;
  auto rows = [&](const void *base, size_t elem, int nrows, size_t row_elems, size_t stride) -> hipError_t {
    for (int r = 0; r < nrows; ++r) {
      hipError_t e = hipMemcpy(dst + (size_t)r * row_elems * elem,
                               (const uint8_t *)base + ((size_t)i * nrows + r) * stride * elem,
                               row_elems * elem, hipMemcpyDeviceToHost);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  };
  hipError_t e = hipSuccess;
  switch (which) {
    case KVQ_TR_SHAT: e = rows(w.shat, 4, s.Hq, T, s.Tmax); break;
    case KVQ_TR_SP: e = rows(w.sp, 4, s.Hq, T, s.Tmax); break;
    case KVQ_TR_MHAT: e = rows(w.mhat, 4, s.Hq, NB, s.NBmax); break;
    case KVQ_TR_LHAT: e = rows(w.Lhat, 4, s.Hq, NB, s.NBmax); break;
    case KVQ_TR_DELTA: e = rows(w.delta, 4, s.Hq, NB, s.NBmax); break;
    case KVQ_TR_M16: e = rows(w.m16, 4, s.Hq, NB, s.NBmax); break;
    case KVQ_TR_L16: e = rows(w.L16, 4, s.Hq, NB, s.NBmax); break;
    case KVQ_TR_WHAT: e = rows(w.What, 4, s.Hq, NB, s.NBmax); break;
    case KVQ_TR_PI: e = rows(w.pi, 4, s.Hq, NB, s.NBmax); break;
    case KVQ_TR_WT: e = rows(w.Wt, 4, s.Hq, NB, s.NBmax); break;
    case KVQ_TR_W16: e = rows(w.W16, 4, s.Hq, NB, s.NBmax); break;
    case KVQ_TR_K0: e = rows(w.k0, 4, 1, s.Hq, s.Hq); break;
    case KVQ_TR_SSIZE: e = rows(w.ssize, 4, 1, s.Hq, s.Hq); break;
    case KVQ_TR_HFLAGS: e = rows(w.hflags, 4, 1, s.Hq, s.Hq); break;
    case KVQ_TR_SSD: e = rows(w.ssd, 8, 1, s.Hq, s.Hq); break;
    case KVQ_TR_EKEY64: e = rows(w.ekey64, 8, 1, s.Hq, s.Hq); break;
    case KVQ_TR_EVAL64: e = rows(w.eval64, 8, 1, s.Hq, s.Hq); break;
    case KVQ_TR_U: e = rows(w.U, 1, s.Hkv, NB, s.NBmax); break;
    case KVQ_TR_V: e = rows(w.V, 1, s.Hkv, NB, s.NBmax); break;
    case KVQ_TR_VH: e = rows(w.vh, 1, s.Hq, NB, s.NBmax); break;
    default: return KVQ_EINVAL;
  }
  HIPCK(ctx, e);
  return KVQ_OK;
}

kvq_status kvq_selftest_exp2k(const float *x, float *y, int64_t n, void *stream) {
  if (!x || !y || n < 0) return KVQ_EINVAL;
  if (n == 0) return KVQ_OK;
  return launch_exp2k(x, y, n, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

kvq_status kvq_selftest_sort(const uint64_t *keys, int64_t n, uint64_t *out, int32_t *path, void *stream) {
  if (!keys || !out || !path || n < 1 || n > MAX_NB) return KVQ_EINVAL;
  return launch_selftest_sort((const unsigned long long *)keys, (int)n, (unsigned long long *)out, path,
                              (hipStream_t)stream) == hipSuccess
             ? KVQ_OK
             : KVQ_EHIP;
}

kvq_status kvq_selftest_launch_shape(int32_t score_wgs, int32_t mix_blocks) {
  if (score_wgs < 0 || (mix_blocks != 0 && mix_blocks != 8 && mix_blocks != 16 && mix_blocks != MIX_CB))
    return KVQ_EINVAL;
  set_score_grid_cap(score_wgs);
  set_mix_chunk_blocks(mix_blocks == 0 ? MIX_CB : mix_blocks);
  return KVQ_OK;
}

kvq_status kvq_selftest_defer_scores(int32_t ppm) {
  if (ppm < -1 || ppm > 1000001) return KVQ_EINVAL;
  g_defer_ppm = ppm < 0 ? DEFER_PPM : ppm;
  return KVQ_OK;
}

kvq_status kvq_selftest_merge_runs(const uint64_t *in, int64_t n, uint64_t *out, int64_t *n_out) {
  if (n < 0 || (n > 0 && (!in || !out)) || !n_out) return KVQ_EINVAL;
  for (int64_t k = 0; k < n; ++k)
    if ((in[k] >> 49) != 0 || (in[k] & 0xffffu) == 0 ||
        ((in[k] >> 16) & 0xffffu) + (in[k] & 0xffffu) > 0xffffu)
      return KVQ_EINVAL;
  std::vector<unsigned long long> ent(in, in + n), m;
  merge_runs(ent, m);
  std::copy(m.begin(), m.end(), out);
  *n_out = (int64_t)m.size();
  return KVQ_OK;
}

}  // extern "C"
