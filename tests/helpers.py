"""Shared helpers of the test-suite (host logic only; no GPU, no method arithmetic)."""
import numpy as np

import kvq_synth as S


def f16_to_f64(a):
    return np.asarray(a, np.uint16).view(np.float16).astype(np.float64)


def oracle_groups(orc, w, layer, seq, K=None, V=None):
    """Tier 1 + ground truth per KV head of one sequence, built by the oracle."""
    if K is None:
        K, V = S.prefill(w, layer, seq)
    groups = []
    for g in range(w.Hkv):
        k16 = np.ascontiguousarray(K[:, g])
        v16 = np.ascontiguousarray(V[:, g])
        groups.append((orc.build_tier1(k16, v16), k16, v16))
    return groups


def true_tv(orc, tr, h, T):
    """Total variation between the softmax of the canonical FP16-key scores and
    the mixed softmax actually used (fp64)."""
    U = tr.U[np.arange(T) // 64]
    x = np.where(U == 1, tr.sp[h], tr.shat[h]).astype(np.float64)
    s = tr.sp[h].astype(np.float64)
    p = np.exp2(s - s.max()); p /= p.sum()
    pt = np.exp2(x - x.max()); pt /= pt.sum()
    return 0.5 * np.abs(p - pt).sum(), p, pt
