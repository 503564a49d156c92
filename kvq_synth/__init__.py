"""Seeded synthetic inputs shaped like the workloads of the subject page
("Runtime-Certified Bounded-Error Quantized Attention", Résultats
expérimentaux: LLaMA 3.1-8B decode at 8K-128K context).

This module only draws numbers: it holds none of the method's arithmetic and
is the one piece shared by the oracle-side tests and the HIP-side tests and
benchmark.  Every draw comes from numpy's PCG64 seeded with
[config id, layer, sequence, tag], so each side regenerates identical inputs.
Values are float32 N(0,1) draws narrowed to binary16 (round to nearest even)
and returned as uint16 bit patterns.

Shapes follow the public Llama-3.1-8B attention layout (32 query heads,
8 KV heads, head dim 128).  The datasets the page evaluates on (PG-19, NIAH,
RULER) and trained weights are not used; these draws stand in for them.
"""
from dataclasses import dataclass, field

import numpy as np

TAG_K, TAG_V, TAG_OUTLIER, TAG_NEEDLE, TAG_TIED, TAG_HOSTILE, TAG_CTX = 0, 1, 2, 3, 4, 5, 6
TAG_Q = 100       # + step
TAG_APPEND = 1000  # + step


def rng(cfg_id, layer, seq, tag):
    return np.random.default_rng([cfg_id, layer, seq, tag])


def to16(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


@dataclass
class Workload:
    cfg_id: int
    name: str
    n_layers: int
    Hq: int
    Hkv: int
    d: int
    ctx: list                      # prefill length per sequence
    n_outlier: int                 # outlier key channels per (layer, KV head)
    outlier_scale: float
    fixed_outliers: tuple = ()     # fixed channel list (config 1)
    needle: bool = False
    tied_heads: tuple = ()         # per sequence: number of near-tied KV heads
    hostile_frac: float = 0.0
    steps: int = 1
    append_before_decode: bool = False
    max_tokens: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def batch(self):
        return len(self.ctx)


def workload(cfg_id):
    """The five workloads (1 = tiny, 2 = 8K single layer, 3 = 4 x 32K with a
    planted needle, 4 = 128K x 32 layers x 16 steps, 5 = adversarial ladder)."""
    if cfg_id == 1:
        return Workload(1, "tiny-1x4q1kv-d64-1k", 1, 4, 1, 64, [1024], 4, 8.0,
                        fixed_outliers=(3, 17, 40, 58), max_tokens=1024 + 64)
    if cfg_id == 2:
        return Workload(2, "llama8b-layer-8k", 1, 32, 8, 128, [8192], 3, 10.0,
                        append_before_decode=True, max_tokens=8192 + 64)
    if cfg_id == 3:
        return Workload(3, "llama8b-layer-4x32k-needle", 1, 32, 8, 128, [32768] * 4, 3, 10.0,
                        needle=True, max_tokens=32768 + 64)
    if cfg_id == 4:
        return Workload(4, "llama8b-32layer-128k-16step", 32, 32, 8, 128, [131072], 3, 10.0,
                        steps=16, append_before_decode=True, max_tokens=131072 + 64)
    if cfg_id == 5:
        r = rng(5, 0, 0, TAG_CTX)
        ctx = [int(x) for x in r.integers(4096, 65536, size=16, endpoint=True)]
        return Workload(5, "ladder-stress-16seq-4k-64k", 1, 32, 8, 128, ctx, 3, 10.0,
                        tied_heads=tuple((0, 2, 4, 8)[i % 4] for i in range(16)),
                        hostile_frac=0.05, max_tokens=65536 + 64)
    raise ValueError(cfg_id)


def outlier_channels(w, layer, g):
    if w.fixed_outliers:
        return np.array(w.fixed_outliers, np.int64)
    return rng(w.cfg_id, layer, g, TAG_OUTLIER).choice(w.d, size=w.n_outlier, replace=False)


def query(w, layer, seq, step):
    """q for one decode step: uint16 [Hq][d], N(0,1)."""
    return to16(rng(w.cfg_id, layer, seq, TAG_Q + step)
                .standard_normal((w.Hq, w.d), dtype=np.float32))


def _keys_f32(w, layer, seq, g, T):
    r = rng(w.cfg_id, layer, seq, TAG_K * 64 + g)
    k = r.standard_normal((T, w.d), dtype=np.float32)
    k[:, outlier_channels(w, layer, g)] *= w.outlier_scale
    return k


def _values_f32(w, layer, seq, g, T):
    r = rng(w.cfg_id, layer, seq, TAG_V * 64 + g)
    return r.standard_normal((T, w.d), dtype=np.float32)


def prefill(w, layer, seq):
    """Prefill K and V of one sequence at one layer: uint16 [T][Hkv][d] each.

    Structure by workload:
      * outliers: n_outlier key channels per (layer, KV head) scaled up;
      * needle (config 3): for each query head h, one block of its KV head
        (distinct blocks within a KV head) holds keys
        0.8 * sqrt(d) * q_h / |q_h| + 0.1 N(0,1), which gives that block most
        of h's softmax mass at the step-0 query;
      * near-tied (config 5): in sequence i, the first tied_heads[i] KV heads
        repeat one base block (N(0,1) with outliers) in every block, plus a
        uniform perturbation of +-0.004 x the channel's scale: block scores
        differ by less than an INT8 step;
      * hostile values (config 5): a share of (token, 32-channel group) cells
        drawn U(-50, 50) instead of N(0,1).
    """
    T = w.ctx[seq]
    K = np.empty((T, w.Hkv, w.d), np.float32)
    V = np.empty((T, w.Hkv, w.d), np.float32)
    q = query(w, layer, seq, 0).view(np.float16).astype(np.float32) if w.needle else None
    G = w.Hq // w.Hkv
    NB = (T + 63) // 64
    for g in range(w.Hkv):
        tied = bool(w.tied_heads) and g < w.tied_heads[seq]
        if tied:
            r = rng(w.cfg_id, layer, seq, TAG_TIED * 64 + g)
            base = r.standard_normal((64, w.d), dtype=np.float32)
            scale = np.ones(w.d, np.float32)
            scale[outlier_channels(w, layer, g)] = w.outlier_scale
            base *= scale
            reps = np.tile(base, (NB, 1))[:T]
            pert = r.uniform(-0.004, 0.004, size=(T, w.d)).astype(np.float32) * scale
            K[:, g, :] = reps + pert
        else:
            K[:, g, :] = _keys_f32(w, layer, seq, g, T)
        V[:, g, :] = _values_f32(w, layer, seq, g, T)
        if w.needle:
            r = rng(w.cfg_id, layer, seq, TAG_NEEDLE * 64 + g)
            blocks = r.choice(T // 64, size=G, replace=False)
            for i in range(G):
                qh = q[g * G + i]
                b = int(blocks[i])
                K[b * 64:(b + 1) * 64, g, :] = (0.8 * np.sqrt(w.d) * qh / np.linalg.norm(qh)
                                                + 0.1 * r.standard_normal((64, w.d), dtype=np.float32))
            w.meta.setdefault("needle_blocks", {})[(layer, seq, g)] = [int(b) for b in blocks]
        if w.hostile_frac > 0:
            r = rng(w.cfg_id, layer, seq, TAG_HOSTILE * 64 + g)
            ng = w.d // 32
            hit = r.random((T, ng)) < w.hostile_frac
            vals = r.uniform(-50.0, 50.0, size=(int(hit.sum()), 32)).astype(np.float32)
            Vg = V[:, g, :].reshape(T, ng, 32)
            Vg[hit] = vals
            V[:, g, :] = Vg.reshape(T, w.d)
    return to16(K), to16(V)


def append_token(w, layer, seq, step):
    """One appended decode token: K, V uint16 [1][Hkv][d] (i.i.d. keys with the
    layer's outlier channels)."""
    r = rng(w.cfg_id, layer, seq, TAG_APPEND + step)
    k = r.standard_normal((1, w.Hkv, w.d), dtype=np.float32)
    for g in range(w.Hkv):
        k[:, g, outlier_channels(w, layer, g)] *= w.outlier_scale
    v = r.standard_normal((1, w.Hkv, w.d), dtype=np.float32)
    return to16(k), to16(v)


def small(cfg_id=90, T=700, Hq=8, Hkv=2, d=128, seed=0, outliers=3, scale=10.0):
    """A small ragged case for CPU-fast parity: T not a multiple of 64."""
    w = Workload(cfg_id, f"small-{Hq}q{Hkv}kv-d{d}-{T}", 1, Hq, Hkv, d, [T], outliers, scale,
                 max_tokens=T + 64)
    w.meta["seed"] = seed
    return w
