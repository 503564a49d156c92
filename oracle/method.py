"""Plain oracle of one certified decode step (test infrastructure only).

Follows "Runtime-Certified Bounded-Error Quantized Attention" (gist.science
technical summary; French section names used throughout):

* Méthodologie §1 (tiered storage): tier 1 = INT8 keys per channel, INT4 values
  per group, scale/offset, per-block error annotations; tier 2 = FP16 ground
  truth; unconditional fallback to exact dense attention.
* Méthodologie §2 (two-term error decomposition): E_key bounds the total
  variation between exact and approximate softmax through the per-token score
  perturbation Delta; E_val is the attention-mass-weighted sum of per-block
  value reconstruction errors eta_b; both computed online, per head, per step.
* Méthodologie §3 (adaptive precision and fallback ladder): INT8 scoring pass
  estimates block mass; top-K* blocks covering tau_cov of it get FP16 keys; the
  INT8 block ranking is checked against the FP16 ranking of the promoted
  blocks; the ladder is (1) widen coverage, (2) promote values, (3) per-head
  dense, (4) per-layer dense.
* Contributions clés: deterministic recovery returns the dense output O_dense
  whenever the certified bounds cannot be met.

The arithmetic primitives (codec, scores, Delta', block ingredients, weights,
fp64 attention) live in oracle.c; this module holds the decisions, which are
integer or fp64 and written here with Python ints and floats (IEEE binary64),
in the order the page gives the steps.  Where the page leaves a step open the
reading is stated at the function; none of it shares code with the HIP path.
"""
import math
from dataclasses import dataclass, field

import numpy as np

from ._lib import lib, ptr, c_array

BLOCK = 64
VGROUP = 32


@dataclass
class Config:
    """Thresholds.  tau_cov = 0.995 is the page's example (Méthodologie §3);
    the others are readings (the page names v_tol but prints no values)."""
    tau_ppm: int = 995_000           # coverage of estimated mass
    eps_key: float = 1e-3            # E_key tolerance (rungs 1 and 3)
    v_tol: float = 0.25              # E_val tolerance (rung 2)
    rho_ppm: int = 900_000           # Spearman threshold of the ranking check
    widen_rounds: int = 2            # R1, rounds of rung 1
    layer_frac_ppm: int = 500_000    # rung 4 when more than this share of heads is at rung 3
    force_dense: bool = False        # every head at level 4 (test hook)
    fp16_values: bool = False        # values in FP16 for every block (the pages' ablation)


# --------------------------------------------------------------------------
# thin wrappers over oracle.c
# --------------------------------------------------------------------------

def h2f(h):
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float32)


def exp2k(x):
    x = c_array(x, np.float32)
    y = np.empty_like(x)
    lib().orc_exp2k_vec(x.size, ptr(x), ptr(y))
    return y


def exp2k_coeffs():
    c = np.empty(8, np.float32)
    lib().orc_exp2k_coeffs(ptr(c))
    return c


def build_tier1(k16, v16):
    """O1 codec over one (sequence, layer, KV head) token stream.
    k16, v16: uint16 fp16 bit patterns [T][d]."""
    k16 = c_array(k16, np.uint16)
    v16 = c_array(v16, np.uint16)
    T, d = k16.shape
    NB = (T + BLOCK - 1) // BLOCK
    t1 = dict(
        T=T, d=d,
        kcode=np.zeros((T, d), np.uint8),
        kscale=np.zeros((NB, d), np.uint16),
        koff=np.zeros((NB, d), np.uint16),
        vcode=np.zeros((T, d), np.uint8),
        vscale=np.zeros((T, d // VGROUP), np.uint16),
        voff=np.zeros((T, d // VGROUP), np.uint16),
        eta=np.zeros(NB, np.float32),
        vmin=np.zeros(d, np.float32),
        vmax=np.zeros(d, np.float32),
    )
    lib().orc_build_tier1(T, d, ptr(k16), ptr(v16), ptr(t1["kcode"]), ptr(t1["kscale"]),
                          ptr(t1["koff"]), ptr(t1["vcode"]), ptr(t1["vscale"]),
                          ptr(t1["voff"]), ptr(t1["eta"]), ptr(t1["vmin"]), ptr(t1["vmax"]))
    return t1


def query(q16):
    """O2: q' = fl32(q * fl32(log2(e)/sqrt(d))), q16 uint16 [G][d]."""
    q16 = c_array(q16, np.uint16)
    G, d = q16.shape
    qp = np.empty((G, d), np.float32)
    lib().orc_query(G, d, ptr(q16), ptr(qp))
    return qp


def int8_scores(qp, t1):
    """O3 + O6: INT8 scores shat [G][T] and per-block Delta' [G][NB]."""
    qp = c_array(qp, np.float32)
    G, d = qp.shape
    T = t1["T"]
    NB = (T + BLOCK - 1) // BLOCK
    shat = np.empty((G, T), np.float32)
    delta = np.empty((G, NB), np.float32)
    lib().orc_int8_scores(G, d, T, ptr(qp), ptr(t1["kcode"]), ptr(t1["kscale"]),
                          ptr(t1["koff"]), ptr(shat), ptr(delta))
    return shat, delta


def fp16_scores(qp, k16):
    """O4: canonical FP16-key scores s' [G][T]."""
    qp = c_array(qp, np.float32)
    k16 = c_array(k16, np.uint16)
    G, d = qp.shape
    T = k16.shape[0]
    sp = np.empty((G, T), np.float32)
    lib().orc_fp16_scores(G, d, T, ptr(qp), ptr(k16), ptr(sp))
    return sp


def ingredients(x):
    """O5: per-block (m_b, L_b) of one score row."""
    x = c_array(x, np.float32)
    T = x.size
    NB = (T + BLOCK - 1) // BLOCK
    m = np.empty(NB, np.float32)
    L = np.empty(NB, np.uint32)
    lib().orc_ingredients(T, ptr(x), ptr(m), ptr(L))
    return m, L


def weights(m, L, mask=None):
    """O7/O10: fixed-point weights relative to the largest block of the set."""
    m = c_array(m, np.float32)
    L = c_array(L, np.uint32)
    NB = m.size
    mk = np.ones(NB, np.uint8) if mask is None else c_array(mask, np.uint8)
    W = np.empty(NB, np.uint32)
    lib().orc_weights(NB, ptr(m), ptr(L), ptr(mk), ptr(W))
    return W


def gfactors(delta):
    delta = c_array(delta, np.float32)
    gp = np.empty(delta.size, np.float64)
    gm = np.empty(delta.size, np.float64)
    lib().orc_gfactors(delta.size, ptr(delta), ptr(gp), ptr(gm))
    return gp, gm


def attend(x, val):
    """fp64 softmax attention with scores x [G][T] (log2 units), values val [T][d]."""
    x = c_array(x, np.float32)
    val = c_array(val, np.float64)
    G, T = x.shape
    d = val.shape[1]
    out = np.empty((G, d), np.float64)
    lib().orc_attend(G, d, T, ptr(x), ptr(val), ptr(out))
    return out


def value_rows(t1, v16, vmask=None):
    """Values an output uses: fp16 on vmask blocks, canonical dequant elsewhere."""
    T, d = t1["T"], t1["d"]
    v16 = c_array(v16, np.uint16)
    val = np.empty((T, d), np.float64)
    vm = None if vmask is None else c_array(vmask, np.uint8)
    lib().orc_value_rows(T, d, ptr(v16), ptr(t1["vcode"]), ptr(t1["vscale"]),
                         ptr(t1["voff"]), ptr(vm), ptr(val))
    return val


# --------------------------------------------------------------------------
# decisions (integers and fp64)
# --------------------------------------------------------------------------

W_UP = 1.0 + 2.0 ** -12
W_DN = 1.0 - 2.0 ** -12


def w_bounds(W):
    """Conservative fp64 bounds on the true mass of each block, in the
    fixed-point unit of W: W- <= mass <= W+.  +65 absorbs the at most 64
    per-token floors of L_b and the floor of W_b; the 2^-12 factors absorb
    the relative error of exp2k and the fp32 products (each ~2^-22)."""
    Wp = [(int(w) + 65) * W_UP for w in W]
    Wm = [int(w) * W_DN for w in W]
    return Wp, Wm


def rank_order(W):
    """pi: blocks sorted by (W descending, index ascending); ties go to the
    lowest block index."""
    return sorted(range(len(W)), key=lambda b: (-int(W[b]), b))


def k_star(W, pi, tau_ppm):
    """Smallest k >= 1 whose top-k blocks hold at least tau_cov of the
    estimated mass: 10^6 * sum_{i<k} W_pi(i) >= tau_ppm * sum_b W_b."""
    total = sum(int(w) for w in W)
    acc = 0
    for k, b in enumerate(pi, start=1):
        acc += int(W[b])
        if 10 ** 6 * acc >= tau_ppm * total:
            return k
    return len(pi)


def ranking_consistent(S_list, W16, rho_ppm):
    """Ranking-consistency check (Méthodologie §3).  Reading: Spearman rank
    correlation between the INT8 ranking of the promoted blocks S_h (their
    order in pi) and their FP16 ranking (W16 descending, index ascending),
    required >= rho_min, evaluated exactly in integers:
        6 * 10^6 * sum d^2 <= (10^6 - rho_ppm) * n (n^2 - 1)."""
    n = len(S_list)
    if n <= 1:
        return True, 0
    r8 = {b: i for i, b in enumerate(S_list)}
    order16 = sorted(S_list, key=lambda b: (-int(W16[b]), b))
    ssd = sum((r8[b] - j) ** 2 for j, b in enumerate(order16))
    return 6 * 10 ** 6 * ssd <= (10 ** 6 - rho_ppm) * n * (n * n - 1), ssd


def e_key(Wt, delta, in_U, gp, gm):
    """E_key (Méthodologie §2): TV(p, p~) <= sum_T P~_b (2^D_b - 1) /
    sum_b P~_b 2^(-D_b [b in T]) with T the INT8 tail (blocks outside U_g).
    Integer sums of ceil/floor of conservative fp64 products; fp64 ratio."""
    Wp, Wm = w_bounds(Wt)
    num = 0
    den = 0
    sub = 0
    for b in range(len(Wt)):
        den += math.floor(Wm[b])
        if not in_U[b]:
            if float(delta[b]) > 20.0:
                return 1.0, None, None
            num += math.ceil(Wp[b] * float(gp[b]))
            sub += math.ceil(Wp[b] * float(gm[b]))
    D = den - sub
    if D <= 0:
        return 1.0, num, D
    return min(1.0, float(num) / float(D)), num, D


def e_val_parts(Wt, eta):
    """Per-block contributions ceil(W+_b eta_b) and the common denominator
    sum_b floor(W-_b) of E_val (Méthodologie §2: mass-weighted eta_b)."""
    Wp, Wm = w_bounds(Wt)
    contrib = [math.ceil(Wp[b] * float(eta[b])) for b in range(len(Wt))]
    den = sum(math.floor(x) for x in Wm)
    return contrib, den


def f32_up(x):
    """fp64 -> fp32 rounded toward +inf (bounds never shrink when reported)."""
    f = np.float32(x)
    if float(f) < x:
        f = np.nextafter(f, np.float32(np.inf))
    return f


@dataclass
class GroupTrace:
    shat: np.ndarray = None
    delta: np.ndarray = None
    sp: np.ndarray = None
    mhat: list = field(default_factory=list)
    Lhat: list = field(default_factory=list)
    m16: list = field(default_factory=list)
    L16: list = field(default_factory=list)
    What: list = field(default_factory=list)
    pi: list = field(default_factory=list)
    k0: list = field(default_factory=list)
    S_size: list = field(default_factory=list)
    Wt: list = field(default_factory=list)
    W16: list = field(default_factory=list)
    ssd: list = field(default_factory=list)
    consistent: list = field(default_factory=list)
    ekey: list = field(default_factory=list)
    eval: list = field(default_factory=list)
    widened: list = field(default_factory=list)
    failed: list = field(default_factory=list)
    V_h: list = field(default_factory=list)
    U: np.ndarray = None
    V: np.ndarray = None
    rounds: int = 0
    level: list = field(default_factory=list)


def group_step(cfg, q16, t1, k16, v16):
    """Decision ladder of one (sequence, layer, KV head) group with G query
    heads (rungs 1-3; rung 4 needs the whole layer and is in decode_step).

    Readings (the page names the rungs but not their triggers):
      * selection is per query head (mass is per head), promotion per KV
        head: U_g is the union of the heads' S_h, and every head of the
        group scores U_g with FP16 keys;
      * each round evaluates every head not yet failed on the current U_g;
        a head whose ranking check fails goes to rung 3 at once; a head with
        E_key > eps_key doubles |S_h| along pi (rung 1) while rounds remain;
        after the last round a head still above eps_key goes to rung 3;
      * rung 2: a head with E_val > v_tol promotes the values of blocks in
        order of contribution (descending, index ascending) until
        E_val <= v_tol; V_g is the union of the heads' V_h.
    """
    G, d = q16.shape
    T = t1["T"]
    NB = (T + BLOCK - 1) // BLOCK
    tr = GroupTrace()
    qp = query(q16)
    tr.shat, tr.delta = int8_scores(qp, t1)
    tr.sp = fp16_scores(qp, k16)
    for h in range(G):
        mh, Lh = ingredients(tr.shat[h])
        m16, L16 = ingredients(tr.sp[h])
        Wh = weights(mh, Lh)
        pi = rank_order(Wh)
        k = k_star(Wh, pi, cfg.tau_ppm)
        tr.mhat.append(mh); tr.Lhat.append(Lh)
        tr.m16.append(m16); tr.L16.append(L16)
        tr.What.append(Wh); tr.pi.append(pi)
        tr.k0.append(k)
    S_size = list(tr.k0)
    failed = [False] * G
    widened = [False] * G
    gpgm = [gfactors(tr.delta[h]) for h in range(G)]
    state = [None] * G
    r = 0
    while True:
        U = np.zeros(NB, np.uint8)
        for h in range(G):
            U[tr.pi[h][:S_size[h]]] = 1
        for h in range(G):
            if failed[h]:
                continue
            m_mix = np.where(U == 1, tr.m16[h], tr.mhat[h]).astype(np.float32)
            L_mix = np.where(U == 1, tr.L16[h], tr.Lhat[h]).astype(np.uint32)
            Wt = weights(m_mix, L_mix)
            S_list = tr.pi[h][:S_size[h]]
            Smask = np.zeros(NB, np.uint8)
            Smask[S_list] = 1
            W16 = weights(tr.m16[h], tr.L16[h], Smask)
            ok, ssd = ranking_consistent(S_list, W16, cfg.rho_ppm)
            ek, _, _ = e_key(Wt, tr.delta[h], U, *gpgm[h])
            state[h] = dict(Wt=Wt, W16=W16, ok=ok, ssd=ssd, ekey=ek)
            if not ok:
                failed[h] = True
        if r == cfg.widen_rounds:
            break
        any_w = False
        for h in range(G):
            if failed[h]:
                continue
            if state[h]["ekey"] > cfg.eps_key and S_size[h] < NB:
                S_size[h] = min(NB, 2 * S_size[h])
                widened[h] = True
                any_w = True
        if not any_w:
            break
        r += 1
    tr.rounds = r
    tr.U = U
    for h in range(G):
        if not failed[h] and state[h]["ekey"] > cfg.eps_key:
            failed[h] = True
    # rung 2: value promotion.  With fp16_values (the FP16-values ablation of
    # Résultats) every block's values come from tier 2 by configuration:
    # V_g = all blocks, no head takes rung 2, and E_val = 0.
    V = np.ones(NB, np.uint8) if cfg.fp16_values else np.zeros(NB, np.uint8)
    contribs = [None] * G
    for h in range(G):
        Vh = []
        if not failed[h]:
            contrib, den = e_val_parts(state[h]["Wt"], t1["eta"])
            contribs[h] = (contrib, den)
            rem = sum(contrib)
            if not cfg.fp16_values and float(rem) / float(den) > cfg.v_tol:
                for b in sorted(range(NB), key=lambda b: (-contrib[b], b)):
                    Vh.append(b)
                    rem -= contrib[b]
                    if float(rem) / float(den) <= cfg.v_tol:
                        break
        tr.V_h.append(sorted(Vh))
        V[Vh] = 1
    tr.V = V
    for h in range(G):
        st = state[h]
        tr.S_size.append(S_size[h])
        tr.Wt.append(st["Wt"]); tr.W16.append(st["W16"])
        tr.ssd.append(st["ssd"]); tr.consistent.append(st["ok"])
        tr.widened.append(widened[h]); tr.failed.append(failed[h])
        if failed[h]:
            tr.ekey.append(0.0); tr.eval.append(0.0)
            tr.level.append(3)
        else:
            contrib, den = contribs[h]
            ev = float(sum(c for b, c in enumerate(contrib) if not V[b])) / float(den)
            tr.ekey.append(st["ekey"]); tr.eval.append(ev)
            tr.level.append(2 if tr.V_h[h] else (1 if widened[h] else 0))
    return tr


def mixed_output(tr, t1, v16):
    """O15 for levels 0-2: FP16-key scores on U_g and INT8 scores elsewhere;
    FP16 values on V_g and dequantized INT4 values elsewhere (fp64)."""
    x = np.where(tr.U[np.arange(t1["T"]) // BLOCK][None, :] == 1, tr.sp, tr.shat)
    val = value_rows(t1, v16, tr.V)
    return attend(x.astype(np.float32), val)


def dense_output(sp, t1, v16):
    """O15 for levels 3-4: dense FP16 attention (canonical FP16-key scores,
    FP16 values, fp64 softmax) -- the exact fallback of Méthodologie §1."""
    val = value_rows(t1, v16, np.ones((t1["T"] + BLOCK - 1) // BLOCK, np.uint8))
    return attend(sp, val)


def naive_output(qp, t1, v16):
    """The uncertified quantized baseline the pages compare against (Résultats:
    naive INT8/INT4 attention): INT8 scores and dequantized INT4 values for
    every token, fp64 softmax; no selection, promotion, bounds or ladder."""
    shat, _ = int8_scores(qp, t1)
    return attend(shat, value_rows(t1, v16))


def dense_attention(q16, k16, v16):
    """Dense attention over FP16 keys and values (Méthodologie §1: the exact
    computation the fallback returns): canonical FP16-key scores, fp64
    softmax and fp64 P.V.  q16 [G][d], k16 and v16 [T][d] (uint16)."""
    sp = fp16_scores(query(q16), k16)
    return attend(sp, h2f(c_array(v16, np.uint16)).astype(np.float64))


@dataclass
class StepResult:
    out: np.ndarray          # [Hq][d] fp64
    e_key: np.ndarray        # [Hq] fp32 (rounded up)
    e_val: np.ndarray        # [Hq] fp32 (rounded up)
    e_key64: list
    e_val64: list
    level: np.ndarray        # [Hq] int8
    groups: list             # GroupTrace per KV head


def decode_step(cfg, q16, groups):
    """One decode step of one sequence at one layer.

    q16: uint16 [Hq][d]; groups: list over KV heads g of (t1, k16, v16), the
    tier-1 arrays and FP16 ground truth of that KV head.  Query heads
    g*G .. g*G+G-1 share KV head g (G = Hq / Hkv).

    Rung 4 (reading): when strictly more than layer_frac of the layer's query
    heads are at rung 3, every head of the layer is recomputed densely.
    """
    Hq, d = q16.shape
    Hkv = len(groups)
    G = Hq // Hkv
    traces = []
    level = np.zeros(Hq, np.int8)
    ek = [0.0] * Hq
    ev = [0.0] * Hq
    for g, (t1, k16, v16) in enumerate(groups):
        tr = group_step(cfg, q16[g * G:(g + 1) * G], t1, k16, v16)
        traces.append(tr)
        for i in range(G):
            level[g * G + i] = tr.level[i]
            ek[g * G + i] = tr.ekey[i]
            ev[g * G + i] = tr.eval[i]
    n3 = int((level == 3).sum())
    if cfg.force_dense or 10 ** 6 * n3 > cfg.layer_frac_ppm * Hq:
        level[:] = 4
    out = np.zeros((Hq, d), np.float64)
    for g, (t1, k16, v16) in enumerate(groups):
        tr = traces[g]
        lv = level[g * G:(g + 1) * G]
        if (lv <= 2).any():
            om = mixed_output(tr, t1, v16)
        if (lv >= 3).any():
            od = dense_output(tr.sp, t1, v16)
        for i in range(G):
            out[g * G + i] = om[i] if lv[i] <= 2 else od[i]
    for h in range(Hq):
        if level[h] >= 3:
            ek[h] = 0.0
            ev[h] = 0.0
    return StepResult(out=out,
                      e_key=np.array([f32_up(x) for x in ek], np.float32),
                      e_val=np.array([f32_up(x) for x in ev], np.float32),
                      e_key64=ek, e_val64=ev, level=level, groups=traces)
