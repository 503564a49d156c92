"""Pins of the oracle's certified bounds, dense fallback and ladder (CPU only).

Page: "Runtime-Certified Bounded-Error Quantized Attention":
  Méthodologie §2 -- E_key bounds the total variation between exact and
  approximate softmax via the per-token score perturbation; E_val is the
  mass-weighted sum of per-block value errors eta_b.
  Méthodologie §1 / Contributions clés -- the fallback is exact dense
  attention, and the ladder returns O_dense when the bounds cannot be met.
  Méthodologie §3 -- the four rungs.
"""
import math

import numpy as np
import pytest
import torch

import kvq_synth as S
from helpers import f16_to_f64, oracle_groups, true_tv


def _group(orc, seed, T=1500, G=1, d=64, qscale=3.0, aligned=False):
    r = np.random.default_rng(seed)
    k = r.standard_normal((T, d)).astype(np.float32)
    k[:, r.choice(d, 3, replace=False)] *= 6
    v = r.standard_normal((T, d)).astype(np.float32)
    q16 = (r.standard_normal((G, d)) * qscale).astype(np.float16).view(np.uint16)
    if aligned:
        # tail keys half a step (0.46) off their code, error sign following q'
        qp = orc.query(q16)[0]
        k = np.clip(k, -1.9, 1.9)
        k16 = k.astype(np.float16).view(np.uint16)
        for b in range(T // 64):
            blk = slice(64 * b, 64 * b + 64)
            kb = k[blk]
            kb[0], kb[1] = -2.0, 2.0
            t1b = orc.build_tier1(kb.astype(np.float16).view(np.uint16), np.zeros((64, d), np.uint16))
            s = f16_to_f64(t1b["kscale"][0])
            j = r.integers(10, 240, size=(64, d))
            frac = np.where((qp > 0)[None, :], 0.46, 0.54)
            x = -2.0 + s[None, :] * (j + frac)
            x[0], x[1] = -2.0, 2.0
            k[blk] = x
    k16 = k.astype(np.float16).view(np.uint16)
    v16 = v.astype(np.float16).view(np.uint16)
    return q16, orc.build_tier1(k16, v16), k16, v16


def test_e_key_closed_form_uniform_delta(orc):
    """All blocks in the tail with the same Delta and mass: the bound equals
    2^(2 Delta) - 2^Delta (up to the conservative margins) and dominates the
    tight worst case tanh(Delta ln2 / 2) of a uniform perturbation."""
    NB = 100
    for D in (1e-4, 0.01, 0.14, 0.7, 3.0):
        Wt = np.full(NB, 2 ** 24, np.uint32)
        delta = np.full(NB, D, np.float32)
        gp, gm = orc.gfactors(delta)
        ek, _, _ = orc.e_key(Wt, delta, np.zeros(NB, np.uint8), gp, gm)
        Dd = float(np.float32(D))
        closed = 2 ** (2 * Dd) - 2 ** Dd
        assert ek >= min(1.0, closed)
        assert ek <= min(1.0, closed * (1 + 1e-3) + 2e-6)
        assert ek >= math.tanh(Dd * math.log(2) / 2)
    # nothing in the tail: zero
    gp, gm = orc.gfactors(np.full(NB, 0.3, np.float32))
    assert orc.e_key(np.full(NB, 2 ** 24, np.uint32), np.full(NB, 0.3, np.float32),
                     np.ones(NB, np.uint8), gp, gm)[0] == 0.0
    # a tail Delta above 20 (log2 units) certifies nothing
    delta = np.full(NB, 0.1, np.float32)
    delta[7] = 21.0
    gp, gm = orc.gfactors(delta)
    assert orc.e_key(np.full(NB, 2 ** 24, np.uint32), delta, np.zeros(NB, np.uint8), gp, gm)[0] == 1.0


CASES = [(s, qs, tau, al) for s in range(4) for qs in (1.0, 3.0) for tau in (900_000, 995_000)
         for al in (False, True)]


@pytest.mark.parametrize("seed,qscale,tau,aligned", CASES)
def test_bounds_dominate_true_errors(orc, seed, qscale, tau, aligned):
    """E_key >= TV(p, p~) and E_val >= |sum_t p~_t (v_t - vbar_t)|_inf, both
    in fp64 against the dense scores; R_v E_key + E_val >= |o~ - o_dense|_inf."""
    d = 64
    q16, t1, k16, v16 = _group(orc, 100 + seed, d=d, qscale=qscale, aligned=aligned)
    cfg = orc.Config(tau_ppm=tau, widen_rounds=0, eps_key=1.0, v_tol=1e9)
    tr = orc.group_step(cfg, q16, t1, k16, v16)
    T = t1["T"]
    tv, p, pt = true_tv(orc, tr, 0, T)
    assert tr.ekey[0] >= tv
    vbar = orc.value_rows(t1, v16, tr.V)
    verr = np.abs(pt @ (f16_to_f64(v16) - vbar)).max()
    assert tr.eval[0] >= verr
    om = orc.mixed_output(tr, t1, v16)[0]
    od = orc.dense_output(tr.sp, t1, v16)[0]
    Rv = float((t1["vmax"].astype(np.float64) - t1["vmin"]).max())
    assert Rv * tr.ekey[0] + tr.eval[0] >= np.abs(om - od).max()


def test_tail_exists_in_bound_cases(orc):
    """The bound cases above exercise a non-empty INT8 tail."""
    q16, t1, k16, v16 = _group(orc, 101, qscale=3.0)
    tr = orc.group_step(orc.Config(tau_ppm=900_000, widen_rounds=0, eps_key=1.0, v_tol=1e9),
                        q16, t1, k16, v16)
    assert 0 < tr.U.sum() < tr.U.size - 4
    assert 0 < tr.ekey[0] < 1


def test_negative_controls_have_teeth(orc):
    """Planting a dropped term in the oracle (on the CPU) breaks the bound
    checks: zero Delta' gives E_key below the true TV; zero eta_b gives E_val
    below the true value error."""
    q16, t1, k16, v16 = _group(orc, 102, qscale=3.0, aligned=True)
    cfg = orc.Config(tau_ppm=900_000, widen_rounds=0, eps_key=1.0, v_tol=1e9)
    real = orc.method.int8_scores
    try:
        orc.method.int8_scores = lambda qp, t: (real(qp, t)[0], np.zeros_like(real(qp, t)[1]))
        tr = orc.group_step(cfg, q16, t1, k16, v16)
    finally:
        orc.method.int8_scores = real
    tv, _, pt = true_tv(orc, tr, 0, t1["T"])
    assert tr.ekey[0] < tv
    t1z = dict(t1, eta=np.zeros_like(t1["eta"]))
    tr = orc.group_step(cfg, q16, t1z, k16, v16)
    _, _, pt = true_tv(orc, tr, 0, t1["T"])
    verr = np.abs(pt @ (f16_to_f64(v16) - orc.value_rows(t1, v16, tr.V))).max()
    assert tr.eval[0] < verr


def test_dense_fallback_is_textbook_attention_and_torch_sdpa(orc):
    w = S.workload(1)
    groups = oracle_groups(orc, w, 0, 0)
    q16 = S.query(w, 0, 0, 0)
    res = orc.decode_step(orc.Config(force_dense=True), q16, groups)
    assert np.all(res.level == 4)
    assert np.all(res.e_key == 0) and np.all(res.e_val == 0)
    k = f16_to_f64(groups[0][1])
    v = f16_to_f64(groups[0][2])
    q = f16_to_f64(q16)
    s = q @ k.T / math.sqrt(w.d)
    p = np.exp(s - s.max(1, keepdims=True))
    ref = (p @ v) / p.sum(1, keepdims=True)
    assert np.abs(res.out - ref).max() < 1e-5
    sd = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(k)[None, None].expand(1, 4, -1, -1),
        torch.from_numpy(v)[None, None].expand(1, 4, -1, -1))
    assert np.abs(res.out - sd[0, :, 0, :].numpy()).max() < 1e-5


def test_full_coverage_and_zero_tolerance_reproduce_dense(orc):
    """tau_cov = 1 and v_tol = 0: every block with nonzero estimated mass gets
    FP16 keys and every block with nonzero eta gets FP16 values, so the output
    is the dense output (Contributions clés: deterministic recovery)."""
    w = S.workload(1)
    groups = oracle_groups(orc, w, 0, 0)
    q16 = S.query(w, 0, 0, 0)
    res = orc.decode_step(orc.Config(tau_ppm=1_000_000, v_tol=0.0), q16, groups)
    dense = orc.decode_step(orc.Config(force_dense=True), q16, groups)
    assert np.all(res.level == 2)
    assert np.abs(res.out - dense.out).max() < 1e-5
    assert np.all(res.e_val == 0)


def test_ladder_near_tied_blocks_fail_ranking(orc):
    """Keys whose block scores differ by less than an INT8 step: the INT8 and
    FP16 rankings disagree, the ranking check fails, the head goes dense
    (rung 3); with every KV head tied, the layer goes dense (rung 4)."""
    w = S.workload(5)
    w.ctx = [4096, 4096]
    w.tied_heads = (2, 8)
    w.hostile_frac = 0.0
    q0 = S.query(w, 0, 0, 0)
    r0 = orc.decode_step(orc.Config(), q0, oracle_groups(orc, w, 0, 0))
    assert np.all(r0.level[:8] == 3) and np.all(r0.level[8:] <= 2)
    assert not any(r0.groups[0].consistent)
    q1 = S.query(w, 0, 1, 0)
    r1 = orc.decode_step(orc.Config(), q1, oracle_groups(orc, w, 0, 1))
    assert np.all(r1.level == 4)


def test_ladder_hostile_values_promote_values(orc):
    w = S.workload(5)
    w.ctx = [4096]
    w.tied_heads = (0,)
    res = orc.decode_step(orc.Config(), S.query(w, 0, 0, 0), oracle_groups(orc, w, 0, 0))
    assert np.all(res.level == 2)
    assert np.all(res.e_val <= 0.25)
    tr = res.groups[0]
    assert 0 < tr.V.sum() <= tr.V.size


def test_ladder_widen_then_dense_when_eps_unreachable(orc):
    q16, t1, k16, v16 = _group(orc, 103, qscale=3.0)
    cfg = orc.Config(tau_ppm=500_000, eps_key=1e-12, v_tol=1e9, widen_rounds=2)
    tr = orc.group_step(cfg, q16, t1, k16, v16)
    assert tr.widened[0] and tr.rounds == 2
    assert tr.S_size[0] == min(tr.U.size, 4 * tr.k0[0])
    assert tr.level[0] == 3
    # with a reachable tolerance the same head stops at rung 1
    cfg = orc.Config(tau_ppm=500_000, eps_key=2e-2, v_tol=1e9, widen_rounds=2)
    tr = orc.group_step(cfg, q16, t1, k16, v16)
    assert tr.level[0] == 1 and tr.ekey[0] <= 2e-2


def test_rung4_when_layer_fraction_is_zero(orc):
    w = S.workload(5)
    w.ctx = [4096]
    w.tied_heads = (1,)
    w.hostile_frac = 0.0
    groups = oracle_groups(orc, w, 0, 0)
    q = S.query(w, 0, 0, 0)
    assert (orc.decode_step(orc.Config(), q, groups).level == 3).sum() == 4
    res = orc.decode_step(orc.Config(layer_frac_ppm=0), q, groups)
    assert np.all(res.level == 4)


def test_needle_block_ranked_first(orc):
    w = S.workload(3)
    w.ctx = [4096]
    groups = oracle_groups(orc, w, 0, 0)
    res = orc.decode_step(orc.Config(), S.query(w, 0, 0, 0), groups)
    G = w.Hq // w.Hkv
    for g in range(w.Hkv):
        tr = res.groups[g]
        needles = w.meta["needle_blocks"][(0, 0, g)]
        for i in range(G):
            assert tr.pi[i][0] == needles[i]
            W = tr.What[i].astype(np.float64)
            assert W[needles[i]] / W.sum() > 0.5


def test_dense_attention_is_textbook_softmax(orc):
    """The dense comparator's definition: softmax(q k^T / sqrt(d)) v over the
    FP16 keys and values, against a plain fp64 numpy evaluation."""
    r = np.random.default_rng(11)
    for T, G, d in ((1, 2, 64), (333, 4, 128)):
        q16 = r.standard_normal((G, d)).astype(np.float16).view(np.uint16)
        k16 = (r.standard_normal((T, d)) * 2).astype(np.float16).view(np.uint16)
        v16 = r.standard_normal((T, d)).astype(np.float16).view(np.uint16)
        q, k, v = f16_to_f64(q16), f16_to_f64(k16), f16_to_f64(v16)
        s = q @ k.T / math.sqrt(d)
        p = np.exp(s - s.max(1, keepdims=True))
        ref = (p @ v) / p.sum(1, keepdims=True)
        assert np.abs(orc.dense_attention(q16, k16, v16) - ref).max() < 1e-5


def test_naive_output_on_grid_equals_dense(orc):
    """Keys on the INT8 grid of their block (scale 2^-5, offset -4, codes 0
    and 255 present per channel) and values on the INT4 grid of their group
    (scale 1/8, offset -1, codes 0 and 15 present): quantization is lossless,
    so the naive INT8/INT4 output equals dense attention up to score
    rounding; on off-grid data it does not (the naive path is uncertified)."""
    r = np.random.default_rng(5)
    T, G, d = 300, 4, 64
    kc = r.integers(0, 256, size=(T, d))
    for b in range(0, T, 64):
        kc[b, :], kc[min(b + 1, T - 1), :] = 0, 255
    vc = r.integers(0, 16, size=(T, d))
    vc[:, 0::32], vc[:, 1::32] = 0, 15
    k = -4.0 + kc / 32.0
    v = -1.0 + vc / 8.0
    k16 = k.astype(np.float16).view(np.uint16)
    v16 = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(f16_to_f64(k16), k) and np.array_equal(f16_to_f64(v16), v)
    t1 = orc.build_tier1(k16, v16)
    assert np.array_equal(t1["kcode"], kc.astype(np.uint8))
    assert np.all(t1["eta"] == 0)
    q16 = r.standard_normal((G, d)).astype(np.float16).view(np.uint16)
    naive = orc.naive_output(orc.query(q16), t1, v16)
    dense = orc.dense_attention(q16, k16, v16)
    assert np.abs(naive - dense).max() < 1e-5
    # off-grid keys: the naive output moves away from dense
    k2 = (r.standard_normal((T, d)) * 3).astype(np.float16).view(np.uint16)
    t2 = orc.build_tier1(k2, v16)
    gap = np.abs(orc.naive_output(orc.query(q16), t2, v16) - orc.dense_attention(q16, k2, v16)).max()
    assert gap > 1e-4


def test_fp16_values_ablation(orc):
    """FP16-values ablation (Résultats): V_g = every block, E_val = 0, no head
    at level 2; with full key coverage the output is the dense output.  On
    hostile values (5 % of groups U(-50, 50)) rung 2 fires without the flag
    and not with it, and the flag's output is closer to dense."""
    w = S.workload(1)
    groups = oracle_groups(orc, w, 0, 0)
    q16 = S.query(w, 0, 0, 0)
    dense = orc.decode_step(orc.Config(force_dense=True), q16, groups)
    res = orc.decode_step(orc.Config(tau_ppm=1_000_000, fp16_values=True), q16, groups)
    assert np.all(res.e_val == 0) and not np.any(res.level == 2)
    assert all(np.all(tr.V == 1) for tr in res.groups)
    assert np.abs(res.out - dense.out).max() < 1e-5

    w5 = S.workload(5)
    w5.ctx, w5.tied_heads, w5.max_tokens = [1500], (0,), 1500 + 64
    g5 = oracle_groups(orc, w5, 0, 0)
    q5 = S.query(w5, 0, 0, 0)
    d5 = orc.decode_step(orc.Config(force_dense=True), q5, g5)
    plain = orc.decode_step(orc.Config(), q5, g5)
    abl = orc.decode_step(orc.Config(fp16_values=True), q5, g5)
    assert np.any(plain.level == 2)
    assert not np.any(abl.level == 2) and np.all(abl.e_val == 0)
    assert np.abs(abl.out - d5.out).max() < np.abs(plain.out - d5.out).max()
