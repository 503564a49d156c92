// kvq_noalloc.hip -- dense FP16 decode attention that allocates nothing.
//
// The same computation and kernels as kvq_dense_decode (split-K chunks of
// the dense decode kernel, then the combine), for callers that cannot
// allocate device memory.  The chunk partials, which kvq_dense_decode keeps
// in a context's scratch, live here in one fixed device array per GPU.
// The array is a file-scope __device__ object: host code cannot pass its
// name to a kernel (that names a host-side stand-in), so its device address
// is resolved once per device with hipGetSymbolAddress and kept per device.
// Every call on one device shares that device's array: two calls whose work
// overlaps on one device race on it.  Every partial a call's combine reads
// is written by the same call first, so nothing needs clearing.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

static __device__ __align__(256) float scratch[KVQ_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_lock;
float *g_ptr[MAX_DEVICES] = {};

thread_local char g_err[256] = "";

kvq_status noalloc_fail(kvq_status st, const char *msg) {
  snprintf(g_err, sizeof(g_err), "%s", msg);
  return st;
}

// Device address of this device's scratch array (resolved on the first call
// on the device, with that device current).
hipError_t scratch_ptr(int dev, float **out) {
  std::lock_guard<std::mutex> lk(g_lock);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = (float *)p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

const char *noalloc_last_error() { return g_err; }

}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_dense_decode_noalloc(int32_t n, int32_t Hq, int32_t Hkv, int32_t d,
                                               int32_t max_tokens, const int32_t *seq_lens,
                                               const void *q, const void *k, const void *v,
                                               float *out, void *stream) {
  g_err[0] = '\0';
  if (n < 1 || n > MAX_CALL || !seq_lens) return noalloc_fail(KVQ_EINVAL, "bad sequence count");
  if (!q || !k || !v || !out) return noalloc_fail(KVQ_EINVAL, "null argument");
  if ((d != 64 && d != 128) || Hkv < 1 || Hkv > 128 || Hq < 1 || Hq % Hkv != 0)
    return noalloc_fail(KVQ_EINVAL, "bad head layout");
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4) return noalloc_fail(KVQ_EINVAL, "bad head layout");
  if (max_tokens < 1 || (max_tokens + BLOCK - 1) / BLOCK > MAX_NB)
    return noalloc_fail(KVQ_EINVAL, "max_tokens out of range");
  DenseArgs a;
  memset(&a, 0, sizeof(a));
  SeqTab tab;
  memset(&tab, 0, sizeof(tab));
  a.n = tab.n = n;
  int maxNB = 0;
  for (int i = 0; i < n; ++i) {
    if (seq_lens[i] < 1 || seq_lens[i] > max_tokens)
      return noalloc_fail(KVQ_EINVAL, "sequence length out of range");
    a.T[i] = tab.T[i] = seq_lens[i];
    tab.nbc[i + 1] = tab.nbc[i] + (seq_lens[i] + BLOCK - 1) / BLOCK;
    maxNB = std::max(maxNB, (seq_lens[i] + BLOCK - 1) / BLOCK);
  }
  Shape s;
  memset(&s, 0, sizeof(s));
  s.L = 1;
  s.Hq = Hq;
  s.Hkv = Hkv;
  s.G = G;
  s.d = d;
  s.nchmax = (maxNB + DEC_CB - 1) / DEC_CB;
  s.NBmax = maxNB;
  s.Tmax = maxNB * BLOCK;
  s.B = n;
  // partials [n][Hkv][nchmax][G][d + 2] floats
  const size_t need = (size_t)n * Hkv * s.nchmax * G * (d + 2) * sizeof(float);
  if (need > KVQ_NOALLOC_SCRATCH_BYTES)
    return noalloc_fail(KVQ_ECAPACITY, "partials exceed the fixed scratch array "
                                       "(KVQ_NOALLOC_SCRATCH_BYTES)");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
    return noalloc_fail(KVQ_EHIP, "no usable current device");
  float *ptr = nullptr;
  if (scratch_ptr(dev, &ptr) != hipSuccess)
    return noalloc_fail(KVQ_EHIP, "hipGetSymbolAddress(scratch) failed");
  Step w;
  memset(&w, 0, sizeof(w));
  w.partd = ptr;
  a.tcap = max_tokens;
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.v = (const uint16_t *)v;
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_dense_vram(s, w, a, maxNB, st);
  if (e == hipSuccess) e = launch_combine(s, w, tab, out, 2, nullptr, nullptr, nullptr, -1, st);
  if (e != hipSuccess) return noalloc_fail(KVQ_EHIP, hipGetErrorString(e));
  return KVQ_OK;
}
