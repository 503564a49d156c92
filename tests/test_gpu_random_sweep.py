"""GPU parity over a seeded sweep of shapes, lengths and thresholds (needs an
MI355X; marked gpu).

Each case draws, from its own seed: 1-3 sequences with ragged lengths
(1-3000 tokens, some with 1-70 appended tokens that cross a block boundary),
a GQA layout, head dim 64 or 128, a query scale (flat to peaked attention,
so K* ranges from a few blocks to all of them) and the controller's
thresholds (coverage, eps_key, v_tol, rho_min, widening rounds), so that the
ladder's paths (widening, value promotion, rung 3, rung 4) all occur across
the sweep.  Every decision-side array is compared bit for bit with the
oracle and every output within max-abs 2e-3 (the shared compare()).  Each
case runs twice: with the INT8 scores stored by the scoring pass, and with
them deferred (the pass stores none; the blocks outside U are rescored after
the selection, in the decode waves of a fused first round or beside the
heads' evaluation, and later rounds read those scores)."""
import numpy as np
import pytest

import kvq_synth as S
from gpu_helpers import Case, compare, log, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

LAYOUTS = [(4, 1), (8, 2), (8, 4), (16, 4), (32, 8), (8, 8), (16, 16)]


@pytest.fixture(scope="module")
def env(orc):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import certified_quantized_kv_amd as kvq
    return kvq, torch, orc


def _sweep_case(seed):
    r = np.random.default_rng(1000 + seed)
    Hq, Hkv = LAYOUTS[int(r.integers(len(LAYOUTS)))]
    d = int(r.choice([64, 128]))
    qscale = float(r.choice([0.5, 1.0, 3.0]))
    cfg = dict(tau_cov_ppm=int(r.choice([900_000, 995_000, 999_999])),
               eps_key=float(r.choice([1e-3, 1e-5])),
               v_tol=float(r.choice([0.25, 0.05])),
               rho_min_ppm=int(r.choice([900_000, 990_000])),
               widen_rounds=int(r.integers(0, 3)))
    rows = []
    for _ in range(int(r.integers(1, 4))):
        T = int(r.integers(1, 3001))
        K = r.standard_normal((T, Hkv, d)).astype(np.float32)
        for g in range(Hkv):
            K[:, g, r.choice(d, 3, replace=False)] *= 10
        V = r.standard_normal((T, Hkv, d)).astype(np.float32)
        q = (r.standard_normal((Hq, d)) * qscale).astype(np.float32)
        ext = None
        if r.random() < 0.5:
            n1 = int(r.integers(1, 71))
            ext = (S.to16(r.standard_normal((n1, Hkv, d)).astype(np.float32)),
                   S.to16(r.standard_normal((n1, Hkv, d)).astype(np.float32)))
        rows.append((S.to16(K), S.to16(V), S.to16(q), ext))
    name = f"sweep-{seed}-{Hq}q{Hkv}kv-d{d}"
    return Case(name, Hq, Hkv, d, rows, **cfg)


@pytest.mark.parametrize("deferred", [False, True], ids=["stored", "deferred"])
@pytest.mark.parametrize("seed", range(16))
def test_random_sweep(env, seed, deferred):
    kvq, torch, orc = env
    case = _sweep_case(seed)
    lens = [s[0].shape[0] + (0 if s[3] is None else s[3][0].shape[0]) for s in case.seqs]
    log(f"[sweep] {case.name} lengths {lens} cfg {case.cfg} deferred {deferred}")
    kvq.set_defer_scores(0 if deferred else 1000001)
    try:
        gpu = run_gpu(kvq, torch, case)
    finally:
        kvq.set_defer_scores(-1)
    assert gpu["stats"]["scores_deferred"] == int(deferred)
    ref = run_oracle(orc, case)
    compare(case, gpu, ref)
    levels = np.concatenate([r.level for r, _ in ref])
    log(f"[sweep] {case.name} levels {np.bincount(levels, minlength=5).tolist()}")
    gpu["ctx"].close()
