/*
 * oracle.c -- plain, slow CPU oracle for certified quantized-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path (the
 * HIP library under certified_quantized_kv_amd/) never links, imports or calls
 * it, and this file shares no code, header, table or constant with it.
 *
 * Subject page: "Runtime-Certified Bounded-Error Quantized Attention"
 * (gist.science technical summary, French and Japanese editions; the two are
 * the same text).  Section names below are those of the French edition:
 *   Méthodologie §1  Stockage à étages            (tier 1 / tier 2 layout)
 *   Méthodologie §2  Décomposition en deux termes (E_key via TV and Delta,
 *                                                   E_val via eta_b and mass)
 *   Méthodologie §3  Précision adaptative et échelle de basculement
 *                                                  (INT8 scoring pass, top-K*,
 *                                                   ranking check, 4 rungs)
 *
 * The page prints no formula, so every arithmetic step below is one reading
 * of it; each reading is listed with its justification in the design notes.
 * Everything that feeds a *decision* (a code, a selection, a verdict, a
 * level) is done in fp32 with IEEE round-to-nearest-even, explicit fmaf, no
 * contraction (build with -ffp-contract=off), so that an independent GPU
 * implementation following the same definition lands on the same bits.
 * Reference outputs are fp64.
 *
 * Compile: gcc -O2 -mfma -ffp-contract=off -fno-fast-math -fPIC -shared
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* fp16 <-> fp32 (bit level, IEEE binary16)                                  */
/* ------------------------------------------------------------------------ */

static inline uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static inline float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* Exact widening of a binary16 value. */
float orc_h2f(uint16_t h)
{
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    if (e == 0) {                       /* zero or subnormal: m * 2^-24 */
        float v = (float)m * 0x1p-24f;  /* exact: m < 2^10 */
        return u2f(f2u(v) | sign);
    }
    if (e == 31) return u2f(sign | 0x7f800000u | (m << 13));
    return u2f(sign | ((e - 15 + 127) << 23) | (m << 13));
}

/* Round-to-nearest-even narrowing to binary16 (finite inputs; overflow -> inf). */
uint16_t orc_f2h(float f)
{
    uint32_t x = f2u(f);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    uint32_t ax = x & 0x7fffffffu;
    if (ax >= 0x7f800000u) return sign | 0x7c00u | (ax > 0x7f800000u ? 0x200u : 0u);
    if (ax >= 0x477ff000u) return sign | 0x7c00u;            /* >= 65520 */
    if (ax < 0x38800000u) {                                   /* < 2^-14   */
        float r = rintf(u2f(ax) * 0x1p24f);                   /* exact scale */
        return sign | (uint16_t)r;                            /* r <= 1024  */
    }
    uint32_t e = (ax >> 23) - 127 + 15, m = ax & 0x7fffffu;
    uint32_t h = (e << 10) | (m >> 13), rem = m & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++;
    return sign | (uint16_t)h;
}

/* Round a non-negative fp32 value to binary16, then step one binary16 ulp up
 * if the result fell below the input: the stored scale never undershoots
 * (reading of "scale" in Méthodologie §1; keeps the round-trip error <= s/2
 * for the scale actually stored). */
uint16_t orc_ru16(float q)
{
    uint16_t h = orc_f2h(q);
    if (orc_h2f(h) < q) h++;
    return h;
}

/* ------------------------------------------------------------------------ */
/* exp2k: the project's own base-2 exponential used by every decision.       */
/* Degree-7 Taylor polynomial of 2^f = e^(f ln 2) on |f| <= 1/2 after        */
/* rounding x to the nearest integer n (Cody-Waite style reduction with the  */
/* base-2 split exact).  c_k = fl32((ln 2)^k / k!).  Results are normal for  */
/* every x >= -125, and exp2k(x) = 0 below that.                              */
/* ------------------------------------------------------------------------ */

static float C_EXP[8];
static int c_exp_ready;

static void init_exp_coeffs(void)
{
    long double t = 1.0L;
    const long double ln2 = 0.693147180559945309417232121458176568L;
    for (int k = 0; k < 8; ++k) {
        C_EXP[k] = (float)t;
        t = t * ln2 / (long double)(k + 1);
    }
    c_exp_ready = 1;
}

void orc_exp2k_coeffs(float *out8)
{
    if (!c_exp_ready) init_exp_coeffs();
    for (int k = 0; k < 8; ++k) out8[k] = C_EXP[k];
}

float orc_exp2k(float x)
{
    if (!c_exp_ready) init_exp_coeffs();
    if (!(x >= -125.0f)) return 0.0f;
    float n = rintf(x);
    float f = x - n;                     /* exact, |f| <= 1/2 */
    float p = C_EXP[7];
    for (int k = 6; k >= 0; --k) p = fmaf(p, f, C_EXP[k]);
    return ldexpf(p, (int)n);
}

void orc_exp2k_vec(int64_t n, const float *x, float *y)
{
    for (int64_t i = 0; i < n; ++i) y[i] = orc_exp2k(x[i]);
}

/* ------------------------------------------------------------------------ */
/* O1  Codec (Méthodologie §1: INT8 keys per channel, INT4 values per group, */
/*     scale/offset metadata, per-block error annotation).                   */
/* ------------------------------------------------------------------------ */

/* Keys of one block (n valid tokens, row stride d), per channel c:
 *   lo/hi = min/max over the block's valid tokens, off = lo,
 *   s = RU16(fl32(hi - lo) / 255)  (0 when hi == lo),
 *   code = clamp(rint(fl32(k - off) / s), 0, 255)  (0 when s == 0). */
void orc_quant_key_block(int n, int d, const uint16_t *k, uint8_t *code,
                         uint16_t *s16, uint16_t *off16)
{
    for (int c = 0; c < d; ++c) {
        float lo = orc_h2f(k[c]), hi = lo;
        for (int t = 1; t < n; ++t) {
            float v = orc_h2f(k[(int64_t)t * d + c]);
            if (v < lo) lo = v;
            if (v > hi) hi = v;
        }
        float r = hi - lo;
        uint16_t sh = (r > 0.0f) ? orc_ru16(r / 255.0f) : 0;
        uint16_t oh = orc_f2h(lo + 0.0f);          /* exact; -0 becomes +0 */
        float s = orc_h2f(sh), off = orc_h2f(oh);
        s16[c] = sh;
        off16[c] = oh;
        for (int t = 0; t < n; ++t) {
            float v = orc_h2f(k[(int64_t)t * d + c]);
            float q = (sh == 0) ? 0.0f : rintf((v - off) / s);
            if (q < 0.0f) q = 0.0f;
            if (q > 255.0f) q = 255.0f;
            code[(int64_t)t * d + c] = (uint8_t)q;
        }
    }
}

/* Values of one token, per group of 32 consecutive channels j:
 *   same rule with 15 levels; returns the token's largest reconstruction
 *   error max_c |fl32(v - fmaf(s, code, off))| (the per-block annotation
 *   eta_b is built from it). */
float orc_quant_value_token(int d, const uint16_t *v, uint8_t *code,
                            uint16_t *s16, uint16_t *off16)
{
    float maxerr = 0.0f;
    for (int j = 0; j < d / 32; ++j) {
        const uint16_t *g = v + 32 * j;
        float lo = orc_h2f(g[0]), hi = lo;
        for (int i = 1; i < 32; ++i) {
            float x = orc_h2f(g[i]);
            if (x < lo) lo = x;
            if (x > hi) hi = x;
        }
        float r = hi - lo;
        uint16_t sh = (r > 0.0f) ? orc_ru16(r / 15.0f) : 0;
        uint16_t oh = orc_f2h(lo + 0.0f);
        float s = orc_h2f(sh), off = orc_h2f(oh);
        s16[j] = sh;
        off16[j] = oh;
        for (int i = 0; i < 32; ++i) {
            float x = orc_h2f(g[i]);
            float q = (sh == 0) ? 0.0f : rintf((x - off) / s);
            if (q < 0.0f) q = 0.0f;
            if (q > 15.0f) q = 15.0f;
            code[32 * j + i] = (uint8_t)q;
            float xhat = fmaf(s, q, off);
            float err = fabsf(x - xhat);
            if (err > maxerr) maxerr = err;
        }
    }
    return maxerr;
}

static inline float nextup_pos(float x) { return u2f(f2u(x) + 1u); }

/* Whole tier 1 of one (sequence, layer, KV head) from its token stream.
 * Plain layouts: kcode[T][d], kscale/koff[NB][d], vcode[T][d] (one code per
 * byte), vscale/voff[T][d/32], eta[NB], vmin/vmax[d].  Blocks are 64 tokens;
 * the last block holds the T mod 64 valid tokens (re-quantized over exactly
 * those, so the result depends only on the token stream). */
void orc_build_tier1(int T, int d, const uint16_t *k, const uint16_t *v,
                     uint8_t *kcode, uint16_t *kscale, uint16_t *koff,
                     uint8_t *vcode, uint16_t *vscale, uint16_t *voff,
                     float *eta, float *vmin, float *vmax)
{
    int NB = (T + 63) / 64;
    for (int b = 0; b < NB; ++b) {
        int t0 = 64 * b, n = (T - t0 < 64) ? T - t0 : 64;
        orc_quant_key_block(n, d, k + (int64_t)t0 * d, kcode + (int64_t)t0 * d,
                            kscale + (int64_t)b * d, koff + (int64_t)b * d);
        float me = 0.0f;
        for (int t = t0; t < t0 + n; ++t) {
            float e = orc_quant_value_token(d, v + (int64_t)t * d, vcode + (int64_t)t * d,
                                            vscale + (int64_t)t * (d / 32),
                                            voff + (int64_t)t * (d / 32));
            if (e > me) me = e;
        }
        eta[b] = (me > 0.0f) ? nextup_pos(me) : 0.0f;
    }
    for (int c = 0; c < d; ++c) {
        float lo = orc_h2f(v[c]), hi = lo;
        for (int t = 1; t < T; ++t) {
            float x = orc_h2f(v[(int64_t)t * d + c]);
            if (x < lo) lo = x;
            if (x > hi) hi = x;
        }
        vmin[c] = lo;
        vmax[c] = hi;
    }
}

/* ------------------------------------------------------------------------ */
/* O2  Query in log2 units: q'_c = fl32(q_c * C), C = fl32(log2(e)/sqrt(d)). */
/* Softmax with natural base and 1/sqrt(d) scaling becomes 2^(q'.k).         */
/* ------------------------------------------------------------------------ */

float orc_query_scale(int d)
{
    return (float)(1.4426950408889634 / sqrt((double)d));
}

void orc_query(int G, int d, const uint16_t *q, float *qp)
{
    float C = orc_query_scale(d);
    for (int i = 0; i < G * d; ++i) qp[i] = orc_h2f(q[i]) * C;
}

/* Per-block dot products over channels (beta and the Delta' sum): one fma
 * chain from 0 over the channels in ascending order,
 *   acc <- fmaf(x_c, y_c, acc)   (x_c replaced by |x_c| when absx is set).
 * Both sides evaluate the chain in exactly this order, so the rounded value
 * is fixed by the definition alone. */
static float chain_dot(int d, const float *x, const float *y, int absx)
{
    float acc = 0.0f;
    for (int c = 0; c < d; ++c)
        acc = fmaf(absx ? fabsf(x[c]) : x[c], y[c], acc);
    return acc;
}

/* ------------------------------------------------------------------------ */
/* O3 + O6  INT8 scoring pass of one block (Méthodologie §3: a lightweight   */
/* pass over the INT8 keys estimates per-block mass) and the per-block bound */
/* on the per-token score perturbation Delta (Méthodologie §2).             */
/*                                                                           */
/* Plain meaning: shat_t = sum_c q'_c (off_c + s_c code_tc).  Canonical:     */
/*   a_c = fl32(q'_c s_c);  e = ilogb(max|a_c|) - 21  (0 if all a_c = 0)      */
/*   A_c = rint(a_c 2^-e)   (|A_c| <= 2^22, an exact integer)                 */
/*   D_t = sum_c A_c (code_tc - 128)        exact integer, any order          */
/*   beta = chain_dot(q', fl32(off + 128 s))   (c ascending, from 0)          */
/*   shat_t = fmaf(fl32(D_t), 2^e, beta)                                      */
/* Delta'_b (log2 units) bounds |shat_t - s'_t| for every valid t, s' being  */
/* the canonical FP16-key score below:                                       */
/*   K'_c = max(|off_c|, |fmaf(256, s_c, off_c)|)                             */
/*   t_c  = fmaf(d 2^-22, K'_c, s_c / 2)                                      */
/*   Delta' = fl32(fl32(chain_dot(|q'|, t) + R) * (1 + 2^-15)),               */
/*   R = 64 d 2^e (0 if all a_c = 0)                                          */
/* s_c/2 is the quantization half-step (Hölder with |q'|), the d 2^-22 K'    */
/* term covers fp32 evaluation error of both score chains, R covers the     */
/* rounding of A, and the final factor covers evaluation of Delta' itself.   */
/* ------------------------------------------------------------------------ */
void orc_int8_block(int G, int d, int n, const float *qp, const uint8_t *code,
                    const uint16_t *s16, const uint16_t *off16,
                    float *shat, int64_t ld_shat, float *delta)
{
    float s[128], off[128], u[128], tt[128], a[128];
    int64_t A[128];
    for (int c = 0; c < d; ++c) {
        s[c] = orc_h2f(s16[c]);
        off[c] = orc_h2f(off16[c]);
        u[c] = fmaf(128.0f, s[c], off[c]);
        float kp = fmaxf(fabsf(off[c]), fabsf(fmaf(256.0f, s[c], off[c])));
        tt[c] = fmaf(ldexpf((float)d, -22), kp, 0.5f * s[c]);
    }
    for (int h = 0; h < G; ++h) {
        const float *q = qp + (int64_t)h * d;
        float amax = 0.0f;
        for (int c = 0; c < d; ++c) {
            a[c] = q[c] * s[c];
            if (fabsf(a[c]) > amax) amax = fabsf(a[c]);
        }
        int zero = (amax == 0.0f);
        int e = zero ? 0 : ilogbf(amax) - 21;
        for (int c = 0; c < d; ++c) A[c] = (int64_t)rintf(ldexpf(a[c], -e));
        float beta = chain_dot(d, q, u, 0);
        float sc = ldexpf(1.0f, e);
        for (int t = 0; t < n; ++t) {
            int64_t D = 0;
            for (int c = 0; c < d; ++c)
                D += A[c] * ((int64_t)code[(int64_t)t * d + c] - 128);
            shat[(int64_t)h * ld_shat + t] = fmaf((float)D, sc, beta);
        }
        float P = chain_dot(d, q, tt, 1);
        float R = zero ? 0.0f : ldexpf(64.0f * (float)d, e);
        delta[h] = (P + R) * (1.0f + 0x1p-15f);
    }
}

/* O4  Canonical FP16-key score: s'_t = fma chain over c ascending of
 * q'_c * k_tc, from 0 (used on promoted blocks and by the dense path). */
void orc_fp16_scores(int G, int d, int T, const float *qp, const uint16_t *k,
                     float *sp /* [G][T] */)
{
    for (int h = 0; h < G; ++h) {
        const float *q = qp + (int64_t)h * d;
        for (int t = 0; t < T; ++t) {
            const uint16_t *kt = k + (int64_t)t * d;
            float acc = 0.0f;
            for (int c = 0; c < d; ++c) acc = fmaf(q[c], orc_h2f(kt[c]), acc);
            sp[(int64_t)h * T + t] = acc;
        }
    }
}

/* INT8 scores and Delta' for all blocks of one group: shat[G][T], delta[G][NB]. */
void orc_int8_scores(int G, int d, int T, const float *qp, const uint8_t *kcode,
                     const uint16_t *kscale, const uint16_t *koff,
                     float *shat, float *delta)
{
    int NB = (T + 63) / 64;
    float dl[8];
    for (int b = 0; b < NB; ++b) {
        int t0 = 64 * b, n = (T - t0 < 64) ? T - t0 : 64;
        orc_int8_block(G, d, n, qp, kcode + (int64_t)t0 * d, kscale + (int64_t)b * d,
                       koff + (int64_t)b * d, shat + t0, T, dl);
        for (int h = 0; h < G; ++h) delta[(int64_t)h * NB + b] = dl[h];
    }
}

/* ------------------------------------------------------------------------ */
/* O5  Block ingredients of a score row x[T] (one head):                     */
/*   m_b = max_t x_t,  L_b = sum_t floor(2^24 exp2k(fl32(x_t - m_b)))        */
/* L_b is an exact integer (<= 2^30), so any summation order agrees.         */
/* ------------------------------------------------------------------------ */
void orc_ingredients(int T, const float *x, float *m, uint32_t *L)
{
    int NB = (T + 63) / 64;
    for (int b = 0; b < NB; ++b) {
        int t0 = 64 * b, t1 = (T < t0 + 64) ? T : t0 + 64;
        float mb = x[t0];
        for (int t = t0 + 1; t < t1; ++t) if (x[t] > mb) mb = x[t];
        uint32_t Lb = 0;
        for (int t = t0; t < t1; ++t)
            Lb += (uint32_t)floorf(0x1p24f * orc_exp2k(x[t] - mb));
        m[b] = mb;
        L[b] = Lb;
    }
}

/* O7/O10  Fixed-point block weights relative to the largest included block:
 *   M = max_{b in set} m_b,  W_b = floor(fl32(fl32(L_b) exp2k(fl32(m_b - M))))
 * for b in the set (mask[b] != 0), 0 elsewhere.  Units of 2^-24. */
void orc_weights(int NB, const float *m, const uint32_t *L, const uint8_t *mask,
                 uint32_t *W)
{
    float M = -INFINITY;
    for (int b = 0; b < NB; ++b) if (mask[b] && m[b] > M) M = m[b];
    for (int b = 0; b < NB; ++b)
        W[b] = mask[b] ? (uint32_t)floorf((float)L[b] * orc_exp2k(m[b] - M)) : 0u;
}

/* O12 helpers: conservative fp64 factors of a tail block's perturbation,
 *   gp >= 2^Delta - 1,   gm >= 1 - 2^-Delta,
 *   gp = fl32(exp2k(Delta) - 1) (1 + 2^-16) + 2^-20  (fp64), likewise gm. */
void orc_gfactors(int n, const float *delta, double *gp, double *gm)
{
    for (int i = 0; i < n; ++i) {
        float up = orc_exp2k(delta[i]) - 1.0f;
        float dn = 1.0f - orc_exp2k(-delta[i]);
        gp[i] = (double)up * (1.0 + 0x1p-16) + 0x1p-20;
        gm[i] = (double)dn * (1.0 + 0x1p-16) + 0x1p-20;
    }
}

/* ------------------------------------------------------------------------ */
/* O15  Attention output in fp64: o_c = sum_t 2^x_t val_tc / sum_t 2^x_t.    */
/* x: [G][T] scores (log2 units), val: [T][d] fp64.                          */
/* ------------------------------------------------------------------------ */
void orc_attend(int G, int d, int T, const float *x, const double *val, double *out)
{
    for (int h = 0; h < G; ++h) {
        const float *xh = x + (int64_t)h * T;
        double mx = -INFINITY;
        for (int t = 0; t < T; ++t) if ((double)xh[t] > mx) mx = xh[t];
        double l = 0.0;
        double acc[128];
        for (int c = 0; c < d; ++c) acc[c] = 0.0;
        for (int t = 0; t < T; ++t) {
            double w = exp2((double)xh[t] - mx);
            l += w;
            const double *vt = val + (int64_t)t * d;
            for (int c = 0; c < d; ++c) acc[c] += w * vt[c];
        }
        for (int c = 0; c < d; ++c) out[(int64_t)h * d + c] = acc[c] / l;
    }
}

/* Value rows used by an output: fp16 ground truth on blocks with vmask[b]
 * set (promoted values), canonical dequant fmaf(s, code, off) elsewhere. */
void orc_value_rows(int T, int d, const uint16_t *v, const uint8_t *vcode,
                    const uint16_t *vscale, const uint16_t *voff,
                    const uint8_t *vmask, double *val)
{
    for (int t = 0; t < T; ++t) {
        int b = t / 64;
        for (int c = 0; c < d; ++c) {
            double x;
            if (vmask && vmask[b]) {
                x = orc_h2f(v[(int64_t)t * d + c]);
            } else {
                int j = c / 32;
                float s = orc_h2f(vscale[(int64_t)t * (d / 32) + j]);
                float off = orc_h2f(voff[(int64_t)t * (d / 32) + j]);
                x = fmaf(s, (float)vcode[(int64_t)t * d + c], off);
            }
            val[(int64_t)t * d + c] = x;
        }
    }
}
