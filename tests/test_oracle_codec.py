"""Pins of the oracle's arithmetic primitives and codec (CPU only).

Page: "Runtime-Certified Bounded-Error Quantized Attention", Méthodologie §1
(INT8 keys per channel, INT4 values per group, scale/offset).  What is pinned
here is fixed by mathematics or by an independent library routine, never by
re-typing the oracle's own formula.
"""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

from helpers import f16_to_f64


def test_h2f_all_patterns_match_numpy(orc):
    L = orc.lib()
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float32)
    got = np.array([L.orc_h2f(int(p)) for p in pats], np.float32)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.all(np.isinf(got[np.isinf(ref)]))


def test_f2h_round_to_nearest_even_matches_numpy(orc):
    L = orc.lib()
    r = np.random.default_rng(1)
    xs = np.concatenate([
        r.standard_normal(20000).astype(np.float32) * 3,
        (r.random(5000) * 1e-4).astype(np.float32),          # f16 subnormal range
        (r.random(5000) * 7e4).astype(np.float32),           # around overflow
        np.array([0.0, -0.0, 65504, 65519.99, 65520, 2 ** -24, 2 ** -25, 3 * 2 ** -26,
                  2 ** -14, 1 + 2 ** -11, 1 + 3 * 2 ** -11], np.float32),
    ])
    # exact ties between two binary16 values
    h = r.integers(0x0400, 0x7bff, 3000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    xs = np.concatenate([xs, ((lo + hi) / 2).astype(np.float32)])
    ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([L.orc_f2h(float(x)) for x in xs], np.uint16)
    assert np.array_equal(got, ref)


def test_ru16_is_smallest_binary16_not_below(orc):
    L = orc.lib()
    r = np.random.default_rng(2)
    qs = np.concatenate([r.random(20000) * 600, r.random(2000) * 1e-6]).astype(np.float32)
    for q in qs:
        h = L.orc_ru16(float(q))
        assert L.orc_h2f(h) >= q
        if h > 0:
            assert L.orc_h2f(h - 1) < q


def _exact_coeff(k):
    getcontext().prec = 60
    ln2 = Decimal(2).ln()
    return ln2 ** k / Decimal(math.factorial(k))


def test_exp2k_coefficients_are_correctly_rounded(orc):
    """c_k = fl32((ln 2)^k / k!): nearest binary32 to the exact value."""
    c = orc.exp2k_coeffs()
    for k in range(8):
        x = _exact_coeff(k)
        f = c[k]
        cands = [np.nextafter(f, np.float32(-1)), f, np.nextafter(f, np.float32(2))]
        dist = [abs(Decimal(float(v)) - x) for v in cands]
        assert dist[1] <= min(dist), (k, f)


def test_exp2k_accuracy_and_special_points(orc):
    r = np.random.default_rng(3)
    x = np.concatenate([r.uniform(-125, 24, 200000), r.uniform(-1, 1, 50000)]).astype(np.float32)
    y = orc.exp2k(x).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    rel = np.abs(y / ref - 1)
    assert rel.max() < 2.0 ** -21
    n = np.arange(-125, 25, dtype=np.float32)
    assert np.array_equal(orc.exp2k(n).astype(np.float64), np.exp2(n.astype(np.float64)))
    assert np.all(orc.exp2k(np.array([-125.5, -200, -np.inf], np.float32)) == 0)
    small = orc.exp2k(np.float32([-125.0, -124.9, -125.0 + 2 ** -10]))
    assert np.all(small >= np.float32(2.0 ** -126))   # always normal when nonzero
    assert orc.exp2k(np.float32([0.0]))[0] == 1.0


def _codec_case(seed, T=1000, d=64):
    r = np.random.default_rng(seed)
    k = r.standard_normal((T, d)).astype(np.float32)
    k[:, [3, 17]] *= 8
    k[:, 40] = 1.5            # constant channel
    v = r.standard_normal((T, d)).astype(np.float32)
    v[5, 0:32] = -0.75        # constant value group
    return k.astype(np.float16).view(np.uint16), v.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("seed,d", [(0, 64), (1, 128)])
def test_key_round_trip_within_half_step(orc, seed, d):
    k16, v16 = _codec_case(seed, d=d)
    t1 = orc.build_tier1(k16, v16)
    T = k16.shape[0]
    blk = np.arange(T) // 64
    s = f16_to_f64(t1["kscale"])[blk]
    off = f16_to_f64(t1["koff"])[blk]
    khat = off + s * t1["kcode"].astype(np.float64)
    err = np.abs(f16_to_f64(k16) - khat)
    assert np.all(err <= s * (0.5 + 2.0 ** -14))
    # scale tight: never more than one binary16 ulp above range/255
    NB = t1["kscale"].shape[0]
    for b in range(NB):
        kb = f16_to_f64(k16[64 * b:64 * b + 64])
        rng_ = kb.max(0) - kb.min(0)
        sb = f16_to_f64(t1["kscale"][b])
        nz = rng_ > 0
        assert np.all(sb[nz] * 255 <= rng_[nz] * (1 + 2.0 ** -9) + 2.0 ** -14)
        assert np.all(sb[~nz] == 0)
        assert np.array_equal(f16_to_f64(t1["koff"][b]), kb.min(0) + 0.0)
        codes = t1["kcode"][64 * b:64 * b + 64]
        assert np.all(codes.min(0) == 0)
        big = (rng_ / 255 >= 2.0 ** -14)
        assert np.all(codes.max(0)[big] == 255)
    # the constant channel reconstructs exactly
    assert np.all(t1["kcode"][:, 40] == 0) and np.all(t1["kscale"][:, 40] == 0)
    assert np.all(khat[:, 40] == 1.5)


def test_value_round_trip_eta_and_ranges(orc):
    k16, v16 = _codec_case(4, d=128)
    t1 = orc.build_tier1(k16, v16)
    T, d = v16.shape
    grp = np.arange(d) // 32
    s = f16_to_f64(t1["vscale"])[:, grp]
    off = f16_to_f64(t1["voff"])[:, grp]
    vhat = off + s * t1["vcode"].astype(np.float64)
    v = f16_to_f64(v16)
    assert np.all(np.abs(v - vhat) <= s * (0.5 + 2.0 ** -14))
    assert t1["vcode"].max() <= 15
    assert np.all(t1["vcode"][5, 0:32] == 0) and np.all(vhat[5, 0:32] == -0.75)
    # eta_b bounds the reconstruction error actually used by the outputs
    used = orc.value_rows(t1, v16)
    blk = np.arange(T) // 64
    err = np.abs(v - used).max(1)
    for b in range(t1["eta"].size):
        eb = err[blk == b].max()
        assert t1["eta"][b] >= eb
        assert t1["eta"][b] <= eb * (1 + 2.0 ** -20) + 1e-30
    assert np.array_equal(t1["vmin"], v.min(0).astype(np.float32))
    assert np.array_equal(t1["vmax"], v.max(0).astype(np.float32))


def test_partial_block_quantized_over_valid_tokens_only(orc):
    """The open last block depends only on its valid tokens: a prefix's tier
    1 equals the full stream's tier 1 on every complete block, and the open
    block equals a one-block quantization of its own tokens."""
    k16, v16 = _codec_case(5, T=1000, d=64)
    full = orc.build_tier1(k16, v16)
    pre = orc.build_tier1(k16[:700], v16[:700])
    assert np.array_equal(pre["kcode"][:640], full["kcode"][:640])
    assert np.array_equal(pre["kscale"][:10], full["kscale"][:10])
    alone = orc.build_tier1(k16[640:700], v16[640:700])
    assert np.array_equal(pre["kcode"][640:700], alone["kcode"])
    assert np.array_equal(pre["kscale"][10], alone["kscale"][0])
    assert np.array_equal(pre["eta"][10], alone["eta"][0])
