// kvq_codec.hip -- quantize-on-append (tier 1 writer) and tier-2 writes.
//
// "Runtime-Certified Bounded-Error Quantized Attention", Méthodologie §1:
// tier 1 keeps INT8 keys per channel and INT4 values per group with
// scale/offset and a per-block error annotation; tier 2 keeps the FP16
// originals.  Readings used here:
//   * key scales/offsets per (64-token block, channel); the open last block
//     is re-quantized over its valid tokens on every append, so tier 1 is a
//     function of the token stream alone;
//   * value groups are 32 consecutive channels of one token (appends never
//     touch older values);
//   * scale = binary16 of range/levels rounded up, offset = the minimum,
//     code = rint((x - offset) / scale) clamped; eta_b = the largest
//     |x - fmaf(scale, code, offset)| over the block's values, one fp32 ulp up.
//
// One workgroup per (sequence, KV head, touched block).  The block's keys
// (old rows from the device copy of the open block, new rows from the
// caller's buffer) and new values are staged in LDS; 64-128 threads own a
// channel each for the key statistics, one thread per (token, value group)
// quantizes values.  New FP16 rows go straight to tier 2 (pinned host memory
// mapped into the device address space), and with resident keys the FP16 keys
// also to their device copy.
//
// The device copy of the open block has two halves.  An append that starts
// inside a partial block reads that block's old rows from half par (the
// workgroup of the first touched block), and the workgroup of the last
// touched block, if it stays partial, writes all of its valid rows to half
// par ^ 1; the host flips par after every append that adds tokens.  When an
// append spans several blocks the two workgroups are different and run in no
// fixed order, so they never touch the same half.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

template <int D>
__global__ __launch_bounds__(256) void k_append(Shape s, Tier1 t, AppendArgs a,
                                                const uint16_t *__restrict__ kin,
                                                const uint16_t *__restrict__ vin) {
  const int i = blockIdx.z, g = blockIdx.y, j = blockIdx.x;
  if (j >= a.n_blk[i]) return;
  const int Told = a.T_old[i], Tnew = Told + a.n_new[i];
  const int b = Told / BLOCK + j, t0 = b * BLOCK;
  const int n = min(BLOCK, Tnew - t0);          // valid rows after the append
  const int r_new = max(Told - t0, 0);          // first new row of the block
  const size_t u = unit_of(s, a.slot[i], a.layer, g);
  const int tid = threadIdx.x;

  __shared__ __align__(16) uint16_t kb[BLOCK][D];
  __shared__ __align__(16) uint16_t vb[BLOCK][D];
  __shared__ __align__(16) uint8_t cb[BLOCK][D];
  __shared__ __align__(16) uint8_t cv[BLOCK][D];
  __shared__ uint32_t s_err;
  if (tid == 0) s_err = 0u;

  const size_t in_row = (size_t)s.Hkv * D;
  for (int idx = tid; idx < BLOCK * (D / 8); idx += 256) {
    const int r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (r < n) {
      if (r < r_new) {
        kv = *(const uint4 *)(t.openk + ((u * 2 + a.par[i]) * BLOCK + r) * D + c8);
      } else {
        const size_t src = (size_t)(a.in_off[i] + t0 + r - Told) * in_row + (size_t)g * D + c8;
        kv = *(const uint4 *)(kin + src);
        vv = *(const uint4 *)(vin + src);
      }
    }
    *(uint4 *)&kb[r][c8] = kv;
    *(uint4 *)&vb[r][c8] = vv;
  }
  __syncthreads();

  // ---- keys: per channel statistics and codes --------------------------------
  if (tid < D) {
    const int c = tid;
    float lo = h2f(kb[0][c]), hi = lo;
    for (int r = 1; r < n; ++r) {
      const float x = h2f(kb[r][c]);
      lo = (x < lo) ? x : lo;
      hi = (x > hi) ? x : hi;
    }
    const float rng = hi - lo;
    const uint16_t sh = (rng > 0.0f) ? ru16(rng / 255.0f) : (uint16_t)0;
    const uint16_t oh = f2h(lo + 0.0f);
    const float sf = h2f(sh), of = h2f(oh);
    t.kmeta[(u * s.NBmax + b) * D + c] = (uint32_t)sh | ((uint32_t)oh << 16);
    for (int r = 0; r < BLOCK; ++r) {
      float qv = 0.0f;
      if (r < n && sh != 0) {
        qv = rintf((h2f(kb[r][c]) - of) / sf);
        qv = fminf(fmaxf(qv, 0.0f), 255.0f);
      }
      cb[r][c] = (uint8_t)qv;
    }
    // running per-channel value range over the new rows
    float vlo = h2f(vb[r_new][c]), vhi = vlo;
    for (int r = r_new + 1; r < n; ++r) {
      const float x = h2f(vb[r][c]);
      vlo = fminf(vlo, x);
      vhi = fmaxf(vhi, x);
    }
    atomicMin(t.vmin + u * D + c, f_ord(vlo));
    atomicMax(t.vmax + u * D + c, f_ord(vhi));
  }

  // ---- values: one thread per (new row, 32-channel group) ----------------------
  constexpr int NG = D / VGROUP;
  float myerr = 0.0f;
  if (tid < (n - r_new) * NG) {
    const int r = r_new + tid / NG, jg = tid % NG;
    const uint16_t *gv = &vb[r][jg * VGROUP];
    float lo = h2f(gv[0]), hi = lo;
    for (int x = 1; x < VGROUP; ++x) {
      const float y = h2f(gv[x]);
      lo = (y < lo) ? y : lo;
      hi = (y > hi) ? y : hi;
    }
    const float rng = hi - lo;
    const uint16_t sh = (rng > 0.0f) ? ru16(rng / 15.0f) : (uint16_t)0;
    const uint16_t oh = f2h(lo + 0.0f);
    const float sf = h2f(sh), of = h2f(oh);
    for (int x = 0; x < VGROUP; ++x) {
      const float y = h2f(gv[x]);
      float qv = 0.0f;
      if (sh != 0) {
        qv = rintf((y - of) / sf);
        qv = fminf(fmaxf(qv, 0.0f), 15.0f);
      }
      cv[r][jg * VGROUP + x] = (uint8_t)qv;
      const float err = fabsf(y - fmaf(sf, qv, of));
      myerr = fmaxf(myerr, err);
    }
    const size_t row = u * s.Tmax + t0 + r;
    t.vmeta[row * NG + jg] = (uint32_t)sh | ((uint32_t)oh << 16);
  }
  if (myerr > 0.0f) atomicMax(&s_err, __float_as_uint(myerr));
  __syncthreads();

  // ---- key codes in MFMA operand order, stored as code ^ 0x80 (the signed
  //      byte code - 128 that the scoring contraction multiplies) -------------
  uint8_t *kdst = t.kcodes + (u * s.NBmax + b) * (size_t)(BLOCK * D);
  for (int q = tid; q < BLOCK * D / 16; q += 256) {
    const int ks = q / 256, nt = (q / 64) % 4, l = q % 64;
    const int r = nt * 16 + (l % 16), c0 = ks * 64 + 16 * (l / 16);
    uint4 x = *(const uint4 *)&cb[r][c0];
    x.x ^= 0x80808080u;
    x.y ^= 0x80808080u;
    x.z ^= 0x80808080u;
    x.w ^= 0x80808080u;
    *(uint4 *)(kdst + (size_t)q * 16) = x;
  }
  // ---- value codes in MFMA operand order (old rows' nibbles kept) --------------
  uint32_t *vdst = (uint32_t *)(t.vcodes + (u * s.NBmax + b) * (size_t)(32 * D));
  for (int q = tid; q < 8 * D; q += 256) {
    const int nt = q >> 7, l = (q >> 1) & 63, qq = q & 1;
    const int c = nt * 16 + (l & 15), rb = 16 * (l >> 4) + 8 * qq;
    const uint32_t old = (r_new > 0) ? vdst[q] : 0u;
    uint32_t word = 0u;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int r = rb + 4 * hi + m, sh = 8 * m + 4 * hi;
        uint32_t nib = 0u;
        if (r < r_new) nib = (old >> sh) & 15u;
        else if (r < n) nib = cv[r][c];
        word |= nib << sh;
      }
    }
    vdst[q] = word;
  }
  // ---- tier 2 (new rows) and the open block's FP16 keys ------------------------
  for (int idx = tid; idx < (n - r_new) * (D / 8); idx += 256) {
    const int r = r_new + idx / (D / 8), c8 = (idx % (D / 8)) * 8;
    const size_t row = u * s.Tmax + t0 + r;
    *(uint4 *)(t.t2k + row * D + c8) = *(const uint4 *)&kb[r][c8];
    *(uint4 *)(t.t2v + row * D + c8) = *(const uint4 *)&vb[r][c8];
    if (t.kres) *(uint4 *)(t.kres + row * D + c8) = *(const uint4 *)&kb[r][c8];
  }
  if (n < BLOCK) {                     // the last touched block stays open
    uint16_t *dst = t.openk + (u * 2 + (a.par[i] ^ 1)) * BLOCK * D;
    for (int idx = tid; idx < n * (D / 8); idx += 256) {
      const int r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
      *(uint4 *)(dst + r * D + c8) = *(const uint4 *)&kb[r][c8];
    }
  }
  if (tid == 0) {
    const float me = __uint_as_float(s_err);
    float e = (me > 0.0f) ? nextup_pos(me) : 0.0f;
    float *ep = t.eta + u * s.NBmax + b;
    if (r_new > 0) e = fmaxf(e, *ep);
    *ep = e;
  }
}

hipError_t launch_append(const Shape &s, const Tier1 &t, const AppendArgs &a, const uint16_t *k,
                         const uint16_t *v, int max_blk, hipStream_t st) {
  if (max_blk <= 0) return hipSuccess;
  dim3 grid(max_blk, s.Hkv, a.n);
  if (s.d == 128)
    return launch_k(k_append<128>, grid, dim3(256), 0, st, s, t, a, k, v);
  else
    return launch_k(k_append<64>, grid, dim3(256), 0, st, s, t, a, k, v);
}

// ---- exports to plain layouts (tests) ---------------------------------------

__global__ void k_export_kcodes(Shape s, Tier1 t, size_t u, int T, uint8_t *dst) {
  const int d = s.d;
  const size_t total = (size_t)T * d;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int tok = (int)(idx / d), c = (int)(idx % d);
    const int b = tok / BLOCK, r = tok % BLOCK;
    const int ks = c / 64, nt = r / 16, l = (r % 16) + 16 * ((c % 64) / 16), jj = c % 16;
    const size_t q = (size_t)((ks * 4 + nt) * 64 + l);
    dst[idx] = t.kcodes[(u * s.NBmax + b) * (size_t)(BLOCK * d) + q * 16 + jj] ^ 0x80u;
  }
}

__global__ void k_export_vcodes(Shape s, Tier1 t, size_t u, int T, uint8_t *dst) {
  const int d = s.d;
  const size_t total = (size_t)T * d;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int tok = (int)(idx / d), c = (int)(idx % d);
    int byte, shift;
    vnib(tok % BLOCK, c, byte, shift);
    const uint8_t v = t.vcodes[(u * s.NBmax + tok / BLOCK) * (size_t)(32 * d) + byte];
    dst[idx] = (v >> shift) & 15;
  }
}

hipError_t launch_export_kcodes(const Shape &s, const Tier1 &t, size_t u, int T, uint8_t *dst,
                                hipStream_t st) {
  return launch_k(k_export_kcodes, dim3(256), dim3(256), 0, st, s, t, u, T, dst);
}
hipError_t launch_export_vcodes(const Shape &s, const Tier1 &t, size_t u, int T, uint8_t *dst,
                                hipStream_t st) {
  return launch_k(k_export_vcodes, dim3(256), dim3(256), 0, st, s, t, u, T, dst);
}

// Copies whole FP16 blocks (64 rows of d halves) between device row arrays:
// entry e of `list` is (source row, destination row) of one block; one
// workgroup per entry, 16-byte loads and stores.  Used by the key block
// cache: cache slot -> staging on a hit, staging -> cache slot on admission.
__global__ __launch_bounds__(256) void k_copy_blocks(const uint32_t *__restrict__ list,
                                                     const uint16_t *__restrict__ src,
                                                     uint16_t *__restrict__ dst, int d) {
  const size_t sr = list[2 * (size_t)blockIdx.x], dr = list[2 * (size_t)blockIdx.x + 1];
  const uint4 *a = reinterpret_cast<const uint4 *>(src + sr * d);
  uint4 *b = reinterpret_cast<uint4 *>(dst + dr * d);
  const int n16 = BLOCK * d / 8;                 // 16-byte words per block
  for (int k = threadIdx.x; k < n16; k += 256) b[k] = a[k];
}

hipError_t launch_copy_blocks(const uint32_t *list, int n, const uint16_t *src, uint16_t *dst,
                              int d, hipStream_t st) {
  if (n < 1) return hipSuccess;
  return launch_k(k_copy_blocks, dim3(n), dim3(256), 0, st, list, src, dst, d);
}

}  // namespace kvq
