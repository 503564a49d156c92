/*
 * kvq.h -- C ABI of the certified quantized-KV decode-attention library
 * (libkvq.so, HIP on AMD Instinct MI355X / gfx950).
 *
 * Method: "Runtime-Certified Bounded-Error Quantized Attention" (gist.science
 * technical summary; French section names are used in citations):
 *   Méthodologie §1  tier 1 in device memory (INT8 keys per channel, INT4
 *                    values per group, scale/offset, per-block error
 *                    annotations); tier 2 = FP16 ground truth in pinned host
 *                    memory; fallback to exact dense attention per head/layer.
 *   Méthodologie §2  per-head, per-step bounds E_key (total variation via the
 *                    per-token score perturbation) and E_val (mass-weighted
 *                    per-block value error), computed without touching FP16.
 *   Méthodologie §3  INT8 scoring pass -> per-block mass -> top-K* blocks
 *                    covering tau_cov promoted to FP16 keys; INT8 vs FP16
 *                    ranking-consistency check; ladder: widen coverage,
 *                    promote values, per-head dense, per-layer dense.
 *
 * Conventions shared by every call:
 *   - Pointers marked (device) are HIP device pointers, (host) are host
 *     pointers.  Arrays are dense, row-major, no padding.
 *   - fp16 data is IEEE binary16 passed as 16-bit words.
 *   - Work is ordered on the caller's `stream` (a hipStream_t passed as
 *     void*; NULL = the null stream).  A call returns once its work is
 *     enqueued; device outputs are valid after the caller synchronises
 *     `stream`.  kvq_decode_step synchronises `stream` internally (it reads
 *     promotion lists and ladder decisions back to issue host->device copies)
 *     and may block the calling thread for that long.
 *   - A context is not thread-safe: use it from one host thread at a time.
 *   - No call throws.  On error the outputs are unspecified; the context
 *     stays usable unless the status is KVQ_EHIP.  kvq_last_error() gives the
 *     message of the last failing call on that context.
 *   - Block size is 64 tokens; value groups are 32 consecutive channels of a
 *     token.  head_dim must be 64 or 128; n_q_heads / n_kv_heads must be 1,
 *     2 or 4; n_kv_heads at most 128.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvq_status;
#define KVQ_OK              0
#define KVQ_EINVAL         -1   /* bad shape, pointer or threshold          */
#define KVQ_ENOMEM_DEVICE  -2   /* device allocation failed                  */
#define KVQ_ENOMEM_HOST    -3   /* pinned host allocation failed (tier 2)    */
#define KVQ_ECAPACITY      -4   /* append past max_tokens                    */
#define KVQ_ESTATE         -5   /* decode on an empty sequence, bad layer    */
#define KVQ_EHIP           -6   /* a HIP runtime error (see kvq_last_error)  */
#define KVQ_ENOTIMPL       -7

#define KVQ_BLOCK_TOKENS   64
#define KVQ_VALUE_GROUP    32
#define KVQ_MAX_CALL_SEQS  64   /* sequences per append/decode call          */

/* flags */
#define KVQ_FLAG_FORCE_DENSE  1u  /* every head at level 4 (exact dense path) */
#define KVQ_FLAG_TIMING       2u  /* fill kvq_step_stats phase times          */
/* FP16 keys kept in device memory (one staging area per (slot, layer, KV
 * head), n_layers * max_batch * n_kv_heads * max_tokens * head_dim * 2 bytes
 * instead of max_batch * n_kv_heads * ...): kvq_append writes each new key to
 * its device copy as well as to tier 2, so promotion copies no keys and the
 * step reads no promotion list back before the FP16 scoring.  Decisions and
 * outputs are unchanged; only host-link traffic, host round trips and the
 * device footprint differ.  Not part of the pages' method (which pages keys
 * in on demand); a device-memory-for-bandwidth trade on GPUs with large
 * HBM. */
#define KVQ_FLAG_RESIDENT_KEYS 4u
/* The pages' FP16-values ablation (Résultats): every block's values are read
 * in FP16 from tier 2 (V_g = all blocks), so E_val = 0 and rung 2 never
 * fires; keys keep the INT8 scoring, selection, ranking check and rungs 1,
 * 3 and 4. */
#define KVQ_FLAG_FP16_VALUES  8u
/* FP16 key blocks promoted in a step are kept in a device cache of
 * key_cache_blocks slots (key_cache_blocks * 64 * head_dim * 2 bytes) shared
 * by all (slot, layer, KV head) units, and later steps take a cached block
 * with a device-to-device copy instead of the host link.  Replacement is least
 * recently used, except that a block used by this call or within the last
 * n_layers calls (one pass over the layers) is never evicted: a promoted
 * block that finds no free slot and no older slot is copied from tier 2
 * without being cached.  kvq_append drops the
 * cached copies of the blocks it changes and kvq_reset_seq those of the
 * sequence.  Decisions and outputs are unchanged.  Not part of the pages'
 * method (a device-memory-for-bandwidth trade within a chosen budget);
 * exclusive with KVQ_FLAG_RESIDENT_KEYS (KVQ_EINVAL if both are set, or if
 * key_cache_blocks < 1 with this flag). */
#define KVQ_FLAG_KEY_CACHE    16u
/* KVQ_FLAG_ALL_SCORES: every step's INT8 pass stores the INT8 scores of every
 * block (the trace KVQ_TR_SHAT then holds them all).  Without it, a step at a
 * layer whose previous step put at least three quarters of the blocks in U
 * stores none in the pass and rescores only the blocks outside U after the
 * selection (the only ones the decode reads); the trace then holds them for
 * those blocks only, and kvq_step_stats.scores_deferred is 1.  Decisions and
 * outputs are the same either way. */
#define KVQ_FLAG_ALL_SCORES   32u

typedef struct kvq_config {
    int32_t n_layers;        /* layers held by the context                      */
    int32_t max_batch;       /* sequence slots 0 .. max_batch-1                 */
    int32_t n_q_heads;       /* query heads per layer                           */
    int32_t n_kv_heads;      /* KV heads per layer (query head h uses KV head
                                h / (n_q_heads / n_kv_heads))                   */
    int32_t head_dim;        /* 64 or 128                                        */
    int32_t max_tokens;      /* capacity per (slot, layer)                       */
    /* thresholds (Méthodologie §3; only tau_cov = 0.995 is the page's example) */
    int32_t tau_cov_ppm;     /* coverage of estimated block mass, ppm (995000)  */
    int32_t rho_min_ppm;     /* Spearman threshold of the ranking check (900000)*/
    int32_t widen_rounds;    /* rounds of rung 1 (2)                             */
    int32_t layer_frac_ppm;  /* rung 4 when more than this share of a layer's
                                query heads is at rung 3, ppm (500000)          */
    double eps_key;          /* E_key tolerance (1e-3)                           */
    double v_tol;            /* E_val tolerance (0.25)                           */
    uint32_t flags;          /* KVQ_FLAG_*                                       */
    int64_t key_cache_blocks;/* slots of the FP16 key block cache
                                (KVQ_FLAG_KEY_CACHE; 0 otherwise)               */
} kvq_config;

/* Fills cfg with the defaults above for the given shape. */
void kvq_default_config(kvq_config *cfg, int32_t n_layers, int32_t max_batch,
                        int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                        int32_t max_tokens);

typedef struct kvq_ctx kvq_ctx;

/* Creates a context on the current HIP device: allocates tier 1 (device),
 * tier 2 (pinned host, 2 * n_layers * max_batch * n_kv_heads * max_tokens *
 * head_dim * 2 bytes) and per-step scratch.  *out is set on success only. */
kvq_status kvq_create(const kvq_config *cfg, kvq_ctx **out);

/* Frees everything the context owns (synchronises the device first). */
void kvq_destroy(kvq_ctx *ctx);

/* Appends tokens to sequences at one layer (Méthodologie §1: quantize into
 * tier 1, keep the FP16 originals in tier 2).
 *   seq_ids (host) [n_seqs]   distinct slots in [0, max_batch)
 *   n_new   (host) [n_seqs]   tokens appended per sequence (>= 0)
 *   k, v    (device) fp16 [sum(n_new)][n_kv_heads][head_dim], sequence i's
 *           tokens first in call order (post-RoPE keys).
 * Re-quantizes the open (partial) last block over its valid tokens, so tier 1
 * depends only on the token stream.  The caller's k/v may be reused once
 * `stream` has passed this call.  KVQ_ECAPACITY if a sequence would exceed
 * max_tokens (nothing is appended then). */
kvq_status kvq_append(kvq_ctx *ctx, int32_t layer, int32_t n_seqs, const int32_t *seq_ids,
                      const int32_t *n_new, const void *k, const void *v, void *stream);

typedef struct kvq_step_stats {
    int64_t promoted_key_blocks;   /* FP16 key blocks copied host->device       */
    int64_t promoted_value_blocks; /* FP16 value blocks copied (rung 2)          */
    int64_t dense_kv_heads;        /* KV heads copied whole for rungs 3/4        */
    int64_t h2d_bytes;             /* bytes copied host->device                  */
    int32_t key_rounds;            /* evaluation rounds of the controller         */
    int32_t host_syncs;            /* host round-trips taken                      */
    int32_t level_count[5];        /* heads per ladder level                      */
    /* times (KVQ_FLAG_TIMING), milliseconds.  Kernel entries are sums of
       kernel durations, each stamped by the runtime at the kernel's own
       start and end (hipExtLaunchKernel events); copies are bracketed by
       events on the copy stream.  The events are recorded only on calls
       that return statistics. */
    float ms_score_int8;           /* INT8 scoring kernel (and the rescoring of a
                                      deferring step, when it has its own launch) */
    float ms_select;               /* top-K* selection, union planning, run lists */
    float ms_score_fp16;           /* FP16 scoring of promoted blocks (all rounds)*/
    float ms_control;              /* controller kernels, all rounds (the first
                                      round is in ms_decode when it shares the
                                      decode's launch, k_eval_decode)             */
    float ms_copy;                 /* host->device copies (copy stream)           */
    float ms_decode;               /* mixed split-K decode kernel (with the first
                                      controller round when they share a launch)  */
    float ms_dense;                /* dense fallback decode kernel                */
    float ms_total;                /* whole call, first launch to last            */
    float ms_combine;              /* split-K combine kernel                      */
    float ms_misc;                 /* rung-4 kernel (only when a head reached
                                      rung 3 or the dense path is forced)         */
    int64_t cached_key_blocks;     /* key blocks taken from the device cache
                                      (KVQ_FLAG_KEY_CACHE), not the host link     */
    int32_t scores_deferred;       /* 1: the INT8 scores were stored for the
                                      blocks outside U only (KVQ_FLAG_ALL_SCORES) */
} kvq_step_stats;

/* One decode step at one layer (Méthodologie §2-§3): attends over every
 * cached token of each sequence (append the step's token first).
 *   seq_ids (host)   [n_seqs] distinct slots, each with >= 1 token at `layer`
 *   q       (device) fp16 [n_seqs][n_q_heads][head_dim]
 *   out     (device) f32  [n_seqs][n_q_heads][head_dim]
 *   e_key   (device) f32  [n_seqs][n_q_heads]  bound on TV(p_dense, p_used)
 *   e_val   (device) f32  [n_seqs][n_q_heads]  bound on the value error,
 *           inf-norm over channels; both 0 for heads at levels 3/4 (exact)
 *   level   (device) int8 [n_seqs][n_q_heads]  0 = certified as selected,
 *           1 = coverage widened, 2 = values promoted, 3 = head dense,
 *           4 = layer dense
 *   stats   (host, nullable) filled before return.
 * Softmax scale is 1/sqrt(head_dim).  With value ranges R_v (per KV head,
 * max over channels of max - min), |out - out_dense|_inf <= R_v * e_key + e_val
 * for levels 0-2, up to fp32 accumulation. */
kvq_status kvq_decode_step(kvq_ctx *ctx, int32_t layer, int32_t n_seqs, const int32_t *seq_ids,
                           const void *q, float *out, float *e_key, float *e_val, int8_t *level,
                           kvq_step_stats *stats, void *stream);

/* Comparators of the certified step (the two reference points of the pages'
 * cost comparison, Résultats: the naive INT8/INT4 baseline and dense
 * attention).  Both reuse the context's per-step scratch, so calls on one
 * context must not overlap any other decode call of that context.
 *
 * kvq_decode_naive: uncertified attention over tier 1 alone -- INT8 scores
 * and dequantized INT4 values for every token, no selection, promotion,
 * bounds or ladder.  Arguments as in kvq_decode_step (seq_ids host, q device
 * fp16 [n_seqs][n_q_heads][head_dim], out device f32 likewise).
 *
 * kvq_dense_decode: standard dense decode attention over an FP16 KV cache
 * that the caller holds in device memory:
 *   seq_lens (host)  [n_seqs], 1 <= seq_lens[i] <= max_tokens (of the config)
 *   q        (device) fp16 [n_seqs][n_q_heads][head_dim]
 *   k, v     (device) fp16 [n_seqs][max_tokens][n_kv_heads][head_dim]; token t
 *            of sequence i at ((i * max_tokens + t) * n_kv_heads + g) * head_dim
 *   out      (device) f32  [n_seqs][n_q_heads][head_dim]
 * Softmax scale 1/sqrt(head_dim); fp32 accumulation.  The context supplies
 * the shape (heads, head_dim, max_tokens, max_batch >= n_seqs) and scratch;
 * its tiers are not read. */
kvq_status kvq_decode_naive(kvq_ctx *ctx, int32_t layer, int32_t n_seqs, const int32_t *seq_ids,
                            const void *q, float *out, void *stream);
kvq_status kvq_dense_decode(kvq_ctx *ctx, int32_t n_seqs, const int32_t *seq_lens, const void *q,
                            const void *k, const void *v, float *out, void *stream);

/* Dense FP16 decode attention that allocates nothing, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same computation and kernels as
 * kvq_dense_decode, without a context:
 *   n_q_heads, n_kv_heads, head_dim   as in kvq_config (head_dim 64 or 128,
 *           n_q_heads / n_kv_heads in {1, 2, 4}, n_kv_heads <= 128)
 *   max_tokens  row capacity of each sequence in k and v
 *   seq_lens (host)  [n_seqs], 1 <= seq_lens[i] <= max_tokens, n_seqs <= 64
 *   q, k, v, out     as in kvq_dense_decode (device; fp16 / f32)
 * The split-K partials live in one fixed device array per GPU of
 * KVQ_NOALLOC_SCRATCH_BYTES, held until the process ends; a call needs
 * n_seqs * n_kv_heads * ceil(ceil(max seq_len / 64) / 8) * (n_q_heads /
 * n_kv_heads) * (head_dim + 2) * 4 bytes of it (at 131072 tokens and 8 KV
 * heads of d = 128: 4.26 MB per sequence) and returns KVQ_ECAPACITY, launching
 * nothing, when that exceeds the array.  The first call on each device
 * resolves the array's address (make it outside graph capture).  Calls whose
 * work overlaps on one device share the array and race.  Stream-ordered on
 * stream.  Errors: the status, and a message in kvq_last_error(NULL) for the
 * calling thread. */
#define KVQ_NOALLOC_SCRATCH_BYTES (16u << 20)
kvq_status kvq_dense_decode_noalloc(int32_t n_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t head_dim, int32_t max_tokens, const int32_t *seq_lens,
                                    const void *q, const void *k, const void *v, float *out,
                                    void *stream);

/* Forgets every token of a slot at every layer.  Synchronises the device
 * first (appends to the slot on any stream complete before its state is
 * cleared) and again before returning. */
kvq_status kvq_reset_seq(kvq_ctx *ctx, int32_t seq_id);

/* Tokens currently held by (slot, layer), or a negative status. */
int64_t kvq_seq_len(const kvq_ctx *ctx, int32_t layer, int32_t seq_id);

const char *kvq_strerror(kvq_status s);
/* Message of the last failing call on ctx; with ctx NULL, of the last
 * failing context-free call (kvq_dense_decode_noalloc) on this thread. */
const char *kvq_last_error(const kvq_ctx *ctx);

/* Device bytes of tier 1 per (token, KV head), and the context's totals. */
double kvq_tier1_bytes_per_token(int32_t head_dim);
int64_t kvq_device_bytes(const kvq_ctx *ctx);
int64_t kvq_host_pinned_bytes(const kvq_ctx *ctx);

/* ---- test and debug exports (parity checks; synchronise the device) ----- */

/* Tier 1 of one (layer, slot, KV head) in plain layouts, written to host_dst
 * as consecutive arrays (T = current length, NB = ceil(T/64), d = head_dim):
 *   kcode  u8  [T][d]          vcode  u8  [T][d] (one code per byte)
 *   kscale u16 [NB][d]         vscale u16 [T][d/32]
 *   koff   u16 [NB][d]         voff   u16 [T][d/32]
 *   eta    f32 [NB]            vmin   f32 [d]      vmax f32 [d]
 * `bytes` must equal kvq_tier1_export_bytes(ctx, layer, seq_id). */
int64_t kvq_tier1_export_bytes(const kvq_ctx *ctx, int32_t layer, int32_t seq_id);
kvq_status kvq_export_tier1(kvq_ctx *ctx, int32_t layer, int32_t seq_id, int32_t kv_head,
                            void *host_dst, size_t bytes);

/* Per-step internals of the last kvq_decode_step for one slot (the arrays of
 * that call; NB = ceil(T/64) of that step, Hq = n_q_heads, Hkv = n_kv_heads).
 * `which` selects one array; shapes are [Hq][T] (scores), [Hq][NB] (block
 * arrays), [Hq] (head arrays), [Hkv][NB] (group block flags). */
#define KVQ_TR_SHAT      1   /* f32 [Hq][T]   INT8 scores (log2 units)              */
#define KVQ_TR_SP        2   /* f32 [Hq][T]   FP16 scores, valid on promoted blocks */
#define KVQ_TR_MHAT      3   /* f32 [Hq][NB]                                         */
#define KVQ_TR_LHAT      4   /* u32 [Hq][NB]                                         */
#define KVQ_TR_DELTA     5   /* f32 [Hq][NB]  score-perturbation bound Delta'        */
#define KVQ_TR_M16       6   /* f32 [Hq][NB]  valid on promoted blocks               */
#define KVQ_TR_L16       7   /* u32 [Hq][NB]  valid on promoted blocks               */
#define KVQ_TR_WHAT      8   /* u32 [Hq][NB]  INT8 block weights                     */
#define KVQ_TR_PI        9   /* u32 [Hq][NB]  blocks by (WHAT desc, index asc)       */
#define KVQ_TR_WT       10   /* u32 [Hq][NB]  final mixed weights                    */
#define KVQ_TR_W16      11   /* u32 [Hq][NB]  final FP16 weights over S_h            */
#define KVQ_TR_K0       12   /* i32 [Hq]      K* of the first round                  */
#define KVQ_TR_SSIZE    13   /* i32 [Hq]      final |S_h|                            */
#define KVQ_TR_SSD      14   /* u64 [Hq]      sum of squared rank differences        */
#define KVQ_TR_EKEY64   15   /* f64 [Hq]      E_key before rounding                  */
#define KVQ_TR_EVAL64   16   /* f64 [Hq]      E_val before rounding                  */
#define KVQ_TR_HFLAGS   17   /* u32 [Hq]      bit0 consistent, bit1 widened, bit2
                                                failed (rung 3), bits 8..15 rounds   */
#define KVQ_TR_U        18   /* u8 [Hkv][NB]  FP16 keys used (union of S_h)          */
#define KVQ_TR_V        19   /* u8 [Hkv][NB]  FP16 values used (union of V_h)        */
#define KVQ_TR_VH       20   /* u8 [Hq][NB]   the head's own value promotions        */
int64_t kvq_trace_bytes(const kvq_ctx *ctx, int32_t which, int32_t seq_id);
kvq_status kvq_export_trace(kvq_ctx *ctx, int32_t which, int32_t seq_id, void *host_dst,
                            size_t bytes);

/* Runs the library's base-2 exponential (the one every decision uses) on n
 * device floats.  For tests. */
kvq_status kvq_selftest_exp2k(const float *x, float *y, int64_t n, void *stream);

/* Sorts n distinct nonzero 64-bit keys into descending order with the
 * workgroup sort that orders the blocks for top-K* selection (weight << 32 |
 * ~block) and for the ranking check (Méthodologie §3): keys and out are
 * device arrays of n entries (1 <= n <= 4096, the blocks of one sequence at
 * most), *path (device int32) receives 0 when the bucket sort placed the keys
 * and 1 when the comparison network (its fallback for clustered keys) sorted
 * them.  Stream-ordered on stream; KVQ_EINVAL on a bad size or null pointer.
 * Duplicate or zero keys are outside the contract.  For tests. */
kvq_status kvq_selftest_sort(const uint64_t *keys, int64_t n, uint64_t *out, int32_t *path,
                             void *stream);

/* Launch shapes of later calls in this process, for determinism tests:
 * score_wgs > 0 caps the workgroups of the INT8 scoring pass (which changes
 * which wave scores which block and which blocks share a batch of channel
 * sums), 0 restores the default; mix_blocks = 8, 16 or 48 sets the most
 * blocks per split-K chunk of the mixed decode (0 = default 48; chunks are
 * cut smaller until the workgroups are a multiple of the compute units).
 * Decisions must not
 * change; outputs differ only by rounding.  Not thread-safe; KVQ_EINVAL on
 * other values.  For tests. */
kvq_status kvq_selftest_launch_shape(int32_t score_wgs, int32_t mix_blocks);

/* When a step stores the INT8 scores only for the blocks outside U
 * (KVQ_FLAG_ALL_SCORES): a step defers them when the previous step at its
 * layer, with its unions read back, had at least ppm parts per million of the
 * call's blocks in U.  ppm = 0 defers every step whose unions are read back,
 * 1000001 none; -1 restores the default 750000.  Decisions and outputs must
 * not change.  Not thread-safe; KVQ_EINVAL on other values.  For tests. */
kvq_status kvq_selftest_defer_scores(int32_t ppm);

/* Merges promotion-plan entries the way a decode step does before copying
 * (host only, no device call).  in: n host entries, each
 * len | start << 16 | group << 32 | kind << 48 (len >= 1, start + len < 2^16,
 * kind 0 or 1); out: host room for n entries, receives the merged entries
 * (overlapping or adjacent runs of one group and kind joined) in (kind,
 * group, start) order, *n_out of them.  KVQ_EINVAL on a malformed entry.
 * For tests. */
kvq_status kvq_selftest_merge_runs(const uint64_t *in, int64_t n, uint64_t *out, int64_t *n_out);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
