"""GPU tests of the deferred INT8 scores (needs an MI355X; marked gpu).

The decode reads the INT8 scores s-hat' only for blocks outside the promoted
union U (inside U it reads the FP16-key scores).  A step may therefore store
no s-hat' in the INT8 pass and rescore the blocks outside U after the
selection; the scores are the same canonical arithmetic either way, so every
decision and output must be bit-identical to a step that stored them all
(KVQ_FLAG_ALL_SCORES), and equal to the oracle's wherever the step defines
them.  The cases lower the coverage target and loosen the tolerances so that
U leaves blocks out and the rescoring has work, on each of its three routes:
the decode waves of a first round fused with the decode (each for its own
blocks), extra workgroups of the evaluation's launch (separate launches), and
a launch of its own (FP16 values: the step starts with the group pass).
"""
import numpy as np
import pytest

import kvq_synth as S
from gpu_helpers import Case, compare, log, run_gpu, run_oracle, same_traces

pytestmark = pytest.mark.gpu

LOOSE = dict(tau_cov_ppm=500_000, eps_key=10.0, v_tol=10.0)


@pytest.fixture(scope="module")
def env(orc):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import certified_quantized_kv_amd as kvq
    return kvq, torch, orc


@pytest.fixture
def defer_all(env):
    kvq = env[0]
    kvq.set_defer_scores(0)
    yield
    kvq.set_defer_scores(-1)


def _seq(cid, T, Hq, Hkv, d):
    w = S.small(cfg_id=cid, T=T, Hq=Hq, Hkv=Hkv, d=d)
    K, V = S.prefill(w, 0, 0)
    return K, V, S.query(w, 0, 0, 0), None


# with FP16 values the step has no first evaluation round of its own (the
# group pass runs from the start), so its decode is not fused with it
@pytest.mark.parametrize("shape", [
    ("700x8x2x128", [(90, 700)], 8, 2, 128, {}),
    ("1500x4x4x64", [(92, 1500)], 4, 4, 64, {}),
    ("ragged-3seq", [(94, 700), (95, 130), (96, 1000)], 8, 2, 128, {}),
    ("700x8x2x128-fp16-values", [(90, 700)], 8, 2, 128, {"fp16_values": True}),
])
def test_deferred_step_matches_oracle(env, defer_all, shape):
    kvq, torch, orc = env
    name, seqs, Hq, Hkv, d, extra = shape
    case = Case(f"deferred {name}", Hq, Hkv, d, [_seq(c, T, Hq, Hkv, d) for c, T in seqs], **LOOSE, **extra)
    log(f"[deferred] {case.name}")
    gpu = run_gpu(kvq, torch, case)
    assert gpu["stats"]["scores_deferred"] == 1
    ref = run_oracle(orc, case)
    outside = sum(int(np.sum(r.groups[g].U == 0)) for r, _ in ref for g in range(Hkv))
    log(f"[deferred] {case.name}: {outside} blocks rescored")
    if not name.startswith("ragged"):
        assert outside > 0, "the case should leave blocks outside U"
    compare(case, gpu, ref)
    gpu["ctx"].close()


def test_deferred_separate_launches_match_oracle(env, defer_all):
    """16-block decode chunks keep the evaluation and the decode in separate
    launches; the evaluation's launch then computes the rescored blocks in
    workgroups of its own, beside the heads."""
    kvq, torch, orc = env
    kvq.set_launch_shape(0, 16)
    try:
        case = Case("deferred separate 700x8x2x128", 8, 2, 128, [_seq(90, 700, 8, 2, 128)], **LOOSE)
        log(f"[deferred] {case.name}")
        gpu = run_gpu(kvq, torch, case)
        assert gpu["stats"]["scores_deferred"] == 1
        ref = run_oracle(orc, case)
        assert sum(int(np.sum(r.groups[g].U == 0)) for r, _ in ref for g in range(2)) > 0
        compare(case, gpu, ref)
        gpu["ctx"].close()
    finally:
        kvq.set_launch_shape(0, 0)


def _run_steps(kvq, torch, K, V, appends, qs, Hq, Hkv, d, cap, layers, **cfg):
    dev = torch.device("cuda:0")
    ctx = kvq.Context(len(set(layers)), 1, Hq, Hkv, d, cap, **cfg)
    for layer in sorted(set(layers)):
        ctx.append(layer, [0], [K.shape[0]], torch.from_numpy(K.view(np.float16)).to(dev),
                   torch.from_numpy(V.view(np.float16)).to(dev))
    res = []
    for layer, (k1, v1), q in zip(layers, appends, qs):
        if k1.shape[0]:
            ctx.append(layer, [0], [k1.shape[0]], torch.from_numpy(k1.view(np.float16)).to(dev),
                       torch.from_numpy(v1.view(np.float16)).to(dev))
        out, ek, ev, lv, st = ctx.decode_step(layer, [0], torch.from_numpy(q[None].view(np.float16)).to(dev),
                                              stats=True)
        torch.cuda.synchronize()
        res.append(dict(out=out.cpu().numpy(), ek=ek.cpu().numpy(), ev=ev.cpu().numpy(),
                        lv=lv.cpu().numpy(), st=st, T=ctx.seq_len(layer, 0),
                        tr={k: ctx.export_trace(k, 0) for k in kvq.TR}))
    ctx.close()
    return res


def _inputs(seed, T, Hq, Hkv, d, sizes):
    # the prefix from the synthetic workload (outlier channels, peaked
    # queries: U leaves blocks out under LOOSE), appends and queries random
    w = S.small(cfg_id=seed, T=T, Hq=Hq, Hkv=Hkv, d=d)
    K, V = S.prefill(w, 0, 0)
    r = np.random.default_rng(seed)
    appends = [((r.standard_normal((n, Hkv, d)) * 2).astype(np.float16).view(np.uint16),
                r.standard_normal((n, Hkv, d)).astype(np.float16).view(np.uint16)) for n in sizes]
    qs = [S.query(w, 0, 0, k) for k in range(len(sizes))]
    return K, V, appends, qs


def _same(a, b, Hq, Hkv):
    for step, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x["out"].view(np.uint32), y["out"].view(np.uint32)), step
        assert np.array_equal(x["lv"], y["lv"]), step
        assert np.array_equal(x["ek"].view(np.uint32), y["ek"].view(np.uint32)), step
        assert np.array_equal(x["ev"].view(np.uint32), y["ev"].view(np.uint32)), step
        same_traces(x["tr"], y["tr"], Hq, Hkv, x["T"], f"step {step}")
        assert x["st"]["promoted_key_blocks"] == y["st"]["promoted_key_blocks"], step


@pytest.mark.parametrize("loose", [False, True])
def test_deferred_bit_identical_over_steps(env, defer_all, loose):
    kvq, torch, _ = env
    Hq, Hkv, d, T = 8, 2, 128, 1000
    sizes = [0, 1, 30, 0, 64]
    K, V, appends, qs = _inputs(31, T, Hq, Hkv, d, sizes)
    cap = T + sum(sizes) + 64
    layers = [0] * len(sizes)
    cfg = LOOSE if loose else {}
    log(f"[deferred] steps, all scores stored (loose={loose})")
    a = _run_steps(kvq, torch, K, V, appends, qs, Hq, Hkv, d, cap, layers, all_scores=True, **cfg)
    log(f"[deferred] steps, scores deferred (loose={loose})")
    b = _run_steps(kvq, torch, K, V, appends, qs, Hq, Hkv, d, cap, layers, **cfg)
    assert all(x["st"]["scores_deferred"] == 0 for x in a)
    assert all(y["st"]["scores_deferred"] == 1 for y in b)
    _same(a, b, Hq, Hkv)


def test_default_policy_follows_last_union(env):
    """Default threshold: a step defers exactly when the previous step at its
    layer had at least 75% of the blocks in U; layers keep separate records."""
    kvq, torch, _ = env
    kvq.set_defer_scores(-1)
    Hq, Hkv, d, T = 4, 4, 64, 1500
    sizes = [0, 1, 0, 2, 0, 3]
    layers = [0, 0, 1, 1, 0, 1]
    for cfg in ({}, LOOSE):
        K, V, appends, qs = _inputs(37, T, Hq, Hkv, d, sizes)
        cap = T + sum(sizes) + 64
        log(f"[deferred] default policy {cfg}")
        a = _run_steps(kvq, torch, K, V, appends, qs, Hq, Hkv, d, cap, layers, all_scores=True, **cfg)
        b = _run_steps(kvq, torch, K, V, appends, qs, Hq, Hkv, d, cap, layers, **cfg)
        _same(a, b, Hq, Hkv)
        last = {}
        for step, (layer, y) in enumerate(zip(layers, b)):
            NB = (y["T"] + 63) // 64
            ppm = int(np.sum(y["tr"]["U"].reshape(Hkv, NB))) * 1_000_000 // (NB * Hkv)
            want = last.get(layer, 0) >= 750_000
            assert y["st"]["scores_deferred"] == int(want), (cfg, step, last)
            last[layer] = ppm
