"""Pins of the oracle's scores, score-perturbation bound Delta', block
ingredients, weights, selection and ranking statistic (CPU only).

Page: "Runtime-Certified Bounded-Error Quantized Attention", Méthodologie §2
(per-token score perturbation Delta) and §3 (INT8 scoring pass, top-K*
covering tau_cov, ranking-consistency check).
"""
import numpy as np
import pytest
import scipy.stats

from helpers import f16_to_f64


def _case(orc, seed, T=900, G=4, d=128, qscale=1.0):
    r = np.random.default_rng(seed)
    k = r.standard_normal((T, d)).astype(np.float32)
    k[:, r.choice(d, 3, replace=False)] *= 10
    v = r.standard_normal((T, d)).astype(np.float32)
    q = (r.standard_normal((G, d)) * qscale).astype(np.float16).view(np.uint16)
    k16 = k.astype(np.float16).view(np.uint16)
    v16 = v.astype(np.float16).view(np.uint16)
    t1 = orc.build_tier1(k16, v16)
    return q, k16, v16, t1


def _exact_scores(orc, q16, k_f64):
    qp = orc.query(q16).astype(np.float64)
    return qp @ k_f64.T, qp


def test_query_scale_is_log2e_over_sqrt_d(orc):
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    for d in (64, 128):
        exact = (Decimal(1) / Decimal(2).ln()) / Decimal(d).sqrt()
        c = np.float32(orc.lib().orc_query_scale(d))
        cands = [np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(1))]
        dist = [abs(Decimal(float(x)) - exact) for x in cands]
        assert dist[1] <= min(dist)


@pytest.mark.parametrize("seed,d", [(0, 128), (1, 64), (2, 128)])
def test_int8_score_matches_dequantized_dot_product(orc, seed, d):
    q16, k16, v16, t1 = _case(orc, seed, d=d)
    T = k16.shape[0]
    blk = np.arange(T) // 64
    khat = (f16_to_f64(t1["koff"])[blk] +
            f16_to_f64(t1["kscale"])[blk] * t1["kcode"].astype(np.float64))
    exact, qp = _exact_scores(orc, q16, khat)
    shat, _ = orc.int8_scores(orc.query(q16), t1)
    scale = np.abs(qp) @ np.abs(khat).T + 1e-30
    assert np.all(np.abs(shat - exact) <= 1e-6 * scale)


@pytest.mark.parametrize("seed,d", [(3, 128), (4, 64)])
def test_fp16_score_within_standard_dot_product_error(orc, seed, d):
    q16, k16, v16, t1 = _case(orc, seed, d=d)
    k = f16_to_f64(k16)
    exact, qp = _exact_scores(orc, q16, k)
    sp = orc.fp16_scores(orc.query(q16), k16)
    gamma = d * 2.0 ** -24 / (1 - d * 2.0 ** -24)
    assert np.all(np.abs(sp - exact) <= gamma * (np.abs(qp) @ np.abs(k).T))


@pytest.mark.parametrize("seed,d,qscale", [(5, 128, 1.0), (6, 64, 1.0), (7, 128, 4.0), (8, 128, 1e-3)])
def test_delta_bounds_score_perturbation(orc, seed, d, qscale):
    """|shat_t - s'_t| <= Delta'_b and |shat_t - exact fp16-key score| <= Delta'_b
    for every token, and Delta' stays within 3 % of the plain Hölder term
    sum_c |q'_c| s_c / 2 (slack terms small)."""
    q16, k16, v16, t1 = _case(orc, seed, d=d, qscale=qscale)
    T = k16.shape[0]
    blk = np.arange(T) // 64
    qp = orc.query(q16)
    shat, delta = orc.int8_scores(qp, t1)
    sp = orc.fp16_scores(qp, k16)
    exact, qp64 = _exact_scores(orc, q16, f16_to_f64(k16))
    D = delta[:, blk].astype(np.float64)
    assert np.all(np.abs(shat - sp) <= D)
    assert np.all(np.abs(shat - exact) <= D)
    holder = np.abs(qp64) @ (f16_to_f64(t1["kscale"]) / 2).T
    assert np.all(delta >= holder)
    assert np.all(delta <= holder * 1.03 + 1e-30)


def test_delta_nearly_tight_on_aligned_rounding(orc):
    """Adversarial block: every key sits half a step off its code with the
    error's sign following q', 0.46 of a step off.  The perturbation then
    reaches >= 85 % of Delta' (a halved bound would fail validity, a doubled
    one this test)."""
    d, n = 128, 64
    r = np.random.default_rng(11)
    q16 = r.standard_normal((1, d)).astype(np.float16).view(np.uint16)
    qp = orc.query(q16)[0]
    base = np.clip(r.standard_normal((n, d)), -1.9, 1.9).astype(np.float32)
    base[0] = -2.0
    base[1] = 2.0                      # fixes every channel's range to [-2, 2]
    k16 = base.astype(np.float16).view(np.uint16)
    t1 = orc.build_tier1(k16, np.zeros((n, d), np.uint16))
    s = f16_to_f64(t1["kscale"][0])
    lo = f16_to_f64(t1["koff"][0])
    j = r.integers(10, 240, size=(n, d))
    # 0.46 of a step above a code rounds down, 0.54 rounds up: the error
    # k - khat then carries the sign of q' in every channel (binary16
    # narrowing moves a value by < 0.04 of a step here)
    frac = np.where((qp > 0)[None, :], 0.46, 0.54)
    x = lo[None, :] + s[None, :] * (j + frac)
    x[0] = -2.0
    x[1] = 2.0
    k16 = x.astype(np.float16).view(np.uint16)
    t1 = orc.build_tier1(k16, np.zeros((n, d), np.uint16))
    shat, delta = orc.int8_scores(orc.query(q16), t1)
    sp = orc.fp16_scores(orc.query(q16), k16)
    err = np.abs(shat[0, 2:] - sp[0, 2:])
    assert err.max() <= delta[0, 0]
    assert err.max() >= 0.85 * delta[0, 0]


def test_block_ingredients_closed_form(orc):
    r = np.random.default_rng(12)
    x = (r.standard_normal(1000) * 5).astype(np.float32)
    x[130:140] = x[130]             # ties
    m, L = orc.ingredients(x)
    for b in range(m.size):
        xb = x[64 * b:64 * b + 64].astype(np.float64)
        assert m[b] == xb.max()
        true = (2.0 ** 24) * np.exp2(xb - xb.max()).sum()
        assert int(L[b]) <= true * (1 + 2.0 ** -20)
        assert true <= (int(L[b]) + 64) * (1 + 2.0 ** -20)


def test_weights_bracket_true_mass(orc):
    """W_b <= 2^24 sum_t 2^(x_t - M) <= (W_b + 65)(1 + 2^-12): the margin the
    bounds rely on."""
    r = np.random.default_rng(13)
    x = (r.standard_normal(64 * 200) * 3).astype(np.float32)
    x[64 * 7:64 * 8] -= 40          # a block far below the max
    m, L = orc.ingredients(x)
    W = orc.weights(m, L)
    M = float(x.max())
    for b in range(m.size):
        true = (2.0 ** 24) * np.exp2(x[64 * b:64 * b + 64].astype(np.float64) - M).sum()
        assert int(W[b]) * orc.method.W_DN <= true <= (int(W[b]) + 65) * orc.method.W_UP
    mask = np.zeros(m.size, np.uint8)
    mask[[3, 9, 50]] = 1
    Wm = orc.weights(m, L, mask)
    assert np.all(Wm[mask == 0] == 0)
    assert Wm[[3, 9, 50]].max() >= 2 ** 24


def test_selection_order_and_kstar_minimal(orc):
    r = np.random.default_rng(14)
    for trial in range(200):
        NB = int(r.integers(1, 60))
        W = r.integers(0, 2 ** 30, NB, dtype=np.int64)
        if trial % 3 == 0:
            W = r.integers(0, 4, NB, dtype=np.int64) * 2 ** 20       # many ties
        W[int(r.integers(NB))] = max(int(W.max()), 2 ** 24)
        tau = int(r.choice([995_000, 900_000, 1_000_000, 500_000]))
        pi = orc.rank_order(W)
        assert pi == list(np.lexsort((np.arange(NB), -W)))        # library sort, ties by index
        k = orc.k_star(W, pi, tau)
        pre = np.cumsum(W[pi])
        ok = [10 ** 6 * int(p) >= tau * int(W.sum()) for p in pre]
        assert ok[k - 1] and not any(ok[:k - 1])


def test_spearman_integer_verdict_matches_library(orc):
    r = np.random.default_rng(15)
    for trial in range(300):
        n = int(r.integers(2, 80))
        S_list = list(r.permutation(200)[:n])
        W16 = np.zeros(200, np.int64)
        noise = r.standard_normal(n) * r.choice([0.01, 0.3, 3.0])
        W16[S_list] = np.maximum(0, (1e6 * (n - np.arange(n) + noise))).astype(np.int64)
        rho_ppm = int(r.choice([900_000, 500_000, 990_000]))
        ok, ssd = orc.ranking_consistent(S_list, W16, rho_ppm)
        r16 = scipy.stats.rankdata(-W16[S_list] + 1e-9 * np.array(S_list), method="ordinal")
        rho = scipy.stats.spearmanr(np.arange(n), r16 - 1).statistic
        exp_ssd = int(((np.arange(n) - (r16 - 1)) ** 2).sum())
        assert ssd == exp_ssd
        if abs(rho - rho_ppm / 1e6) > 1e-12:
            assert ok == (rho >= rho_ppm / 1e6)
    assert orc.ranking_consistent([5], np.ones(6, np.int64), 999_999)[0]


@pytest.mark.parametrize("d", [64, 128])
def test_channel_sums_are_ascending_fma_chains(orc, d):
    """beta and the Delta' sum are fma chains over the channels in ascending
    order from 0 (Méthodologie §2/§3 readings; the order fixes the rounding).
    Closed form by absorption: keys constant per channel (scale 0, offset =
    the value), channel 0 holds 1024, every other channel 2^-15, q = 1, so
    q' = C = fl32(log2(e)/sqrt(d)).  In the ascending chain the first term
    C*1024 is exact and every later term C*2^-15 is below half an ulp of it,
    so beta = C*1024 exactly; any order that adds the small terms first (a
    tree, a reversed chain, the exact sum) lands at least one ulp higher.
    The same holds for Delta': t_0 = d 2^-22 1024, t_c = d 2^-22 2^-15, so
    the chain is C*t_0 and Delta' = fl32(C t_0 (1 + 2^-15))."""
    from fractions import Fraction as Fr
    T = 64
    k = np.full((T, d), 2.0 ** -15, np.float32)
    k[:, 0] = 1024.0
    k16 = k.astype(np.float16).view(np.uint16)
    assert np.array_equal(k16.view(np.float16).astype(np.float32), k)
    v16 = np.zeros((T, d), np.float16).view(np.uint16)
    q16 = np.ones((1, d), np.float16).view(np.uint16)
    t1 = orc.build_tier1(k16, v16)
    assert not t1["kscale"].any()
    qp = orc.query(q16)
    C = np.float32(orc.lib().orc_query_scale(d))
    assert np.all(qp == C)
    shat, delta = orc.int8_scores(qp, t1)

    def half_ulp(x):
        return Fr(2) ** (int(np.floor(np.log2(float(x)))) - 24)
    big, small = Fr(float(C)) * 1024, Fr(float(C)) * Fr(2) ** -15
    assert small < half_ulp(big)                       # each later term absorbed
    assert (d - 1) * small > 2 * half_ulp(big)         # but not their sum
    beta = np.float32(C) * np.float32(1024.0)           # exact: a power-of-two scaling
    assert np.all(shat.view(np.uint32) == beta.view(np.uint32))
    exact = np.float32(float(big + (d - 1) * small))
    assert exact != beta                               # the case tells the orders apart

    t0, ts = Fr(d) * Fr(2) ** -22 * 1024, Fr(d) * Fr(2) ** -22 * Fr(2) ** -15
    p_big, p_small = Fr(float(C)) * t0, Fr(float(C)) * ts
    assert p_small < half_ulp(p_big) and (d - 1) * p_small > 2 * half_ulp(p_big)
    P = np.float32(float(p_big))
    assert Fr(float(P)) == p_big                        # C t_0 is exact
    want = np.float32(P * np.float32(1.0 + 2.0 ** -15))
    assert delta.view(np.uint32)[0, 0] == want.view(np.uint32)


def test_f32_up_is_smallest_float_at_or_above(orc):
    """The fp64 -> binary32 rounding of every reported bound goes up: the
    result is >= x and its binary32 predecessor is < x (so it is the least
    such float), on random values, exact floats, ties and edge cases."""
    from fractions import Fraction as Fr
    r = np.random.default_rng(11)
    xs = list(r.random(2000)) + list(10.0 ** r.uniform(-45, 38, 2000))
    fl = r.random(500).astype(np.float32)
    xs += [float(f) for f in fl]                                   # exactly representable
    xs += [float(f) + float(np.spacing(f)) / 2 for f in fl]        # exact ties
    xs += [float(f) + float(np.spacing(f)) * 1e-6 for f in fl]     # just above a float
    xs += [0.0, 2.0 ** -149, 2.0 ** -150, 3 * 2.0 ** -150, 2.0 ** -126, 1.0, 1.0 - 2.0 ** -60,
           1.0 + 2.0 ** -60, float(np.finfo(np.float32).max)]
    for x in xs:
        f = orc.f32_up(x)
        assert isinstance(f, np.float32)
        assert Fr(float(f)) >= Fr(x), x
        prev = np.nextafter(f, np.float32(-np.inf))
        assert Fr(float(prev)) < Fr(x) or (x == 0.0 and f == 0.0), x
