"""GPU parity: the HIP path through the C ABI against the oracle, element by
element, on the same seeded inputs (needs an MI355X; marked gpu).

Covers: the decision exponential; tier 1 after bulk and piecewise appends
(append equivalence, ragged last block); the whole decode step (every
intermediate array, verdicts, bounds, levels, outputs) on the tiny case, a
ragged multi-KV-head case, the 8K Llama-shaped layer with an appended token,
a multi-sequence needle case, and the ladder cases (near-tied keys, hostile
values, forced widening, rung 4, forced dense); determinism on re-run; ABI
error statuses.
"""
import numpy as np
import pytest

import kvq_synth as S
from gpu_helpers import Case, compare, compare_tier1, f32bits, log, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env(orc):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import certified_quantized_kv_amd as kvq
    return kvq, torch, orc


def _wl_case(w, seqs, name=None, extra=False, **cfg):
    rows = []
    for s in seqs:
        K, V = S.prefill(w, 0, s)
        ext = S.append_token(w, 0, s, 0) if extra else None
        rows.append((K, V, S.query(w, 0, s, 0), ext))
    return Case(name or w.name, w.Hq, w.Hkv, w.d, rows, max_tokens=w.max_tokens, **cfg)


def _random_case(name, T, Hq, Hkv, d, seed, qscale=1.0, n_seqs=1, **cfg):
    r = np.random.default_rng(seed)
    rows = []
    for _ in range(n_seqs):
        K = r.standard_normal((T, Hkv, d)).astype(np.float32)
        for g in range(Hkv):
            K[:, g, r.choice(d, 3, replace=False)] *= 10
        V = r.standard_normal((T, Hkv, d)).astype(np.float32)
        q = (r.standard_normal((Hq, d)) * qscale).astype(np.float32)
        rows.append((S.to16(K), S.to16(V), S.to16(q), None))
    return Case(name, Hq, Hkv, d, rows, **cfg)


def _check(env, case, **kw):
    kvq, torch, orc = env
    log(f"[parity] {case.name}: GPU")
    gpu = run_gpu(kvq, torch, case, **kw)
    log(f"[parity] {case.name}: oracle")
    ref = run_oracle(orc, case)
    compare(case, gpu, ref)
    return gpu, ref


def test_exp2k_bit_exact(env):
    kvq, torch, orc = env
    log("[parity] exp2k")
    r = np.random.default_rng(0)
    x = np.concatenate([r.uniform(-130, 24, 400000), r.uniform(-1, 1, 100000),
                        np.arange(-126, 25, 0.25)]).astype(np.float32)
    y = kvq.exp2k(torch.from_numpy(x).cuda()).cpu().numpy()
    assert np.array_equal(f32bits(y), f32bits(orc.exp2k(x)))


@pytest.mark.parametrize("chunks", [None, [1, 1, 62, 1, 64, 5, 200, 63, 64, 3]])
def test_tier1_matches_oracle(env, chunks):
    """Bulk append and piecewise appends (open block re-quantized each time)
    both give the oracle's tier 1 bit for bit."""
    kvq, torch, orc = env
    case = _random_case("tier1", 700, 8, 2, 128, 3)
    log(f"[parity] tier1 chunks={chunks}")
    gpu = run_gpu(kvq, torch, case, chunks=chunks)
    K, V = case.seqs[0][0], case.seqs[0][1]
    for g in range(case.Hkv):
        t1 = orc.build_tier1(np.ascontiguousarray(K[:, g]), np.ascontiguousarray(V[:, g]))
        compare_tier1(gpu["ctx"], t1, 0, 0, g, f"tier1 kv {g}")
    gpu["ctx"].close()


def test_tier1_multi_sequence_appends_spanning_blocks(env):
    """Appends that start inside an open block and end in another partial
    block, for several sequences in one call whose open-block parities
    differ (each has had a different number of appends): tier 1 equals the
    oracle's for every sequence and KV head."""
    kvq, torch, orc = env
    dev = torch.device("cuda:0")
    r = np.random.default_rng(21)
    T = [300, 257, 190]
    Hkv, d = 2, 128
    K = [S.to16(r.standard_normal((t, Hkv, d)).astype(np.float32) * 3) for t in T]
    V = [S.to16(r.standard_normal((t, Hkv, d)).astype(np.float32)) for t in T]
    sched = [{0: 37, 1: 100, 2: 1}, {0: 90}, {0: 70, 1: 64, 2: 129}, {1: 5, 2: 30},
             {0: 103, 1: 88, 2: 30}]
    ctx = kvq.Context(1, 3, 8, Hkv, d, 320)
    pos = [0, 0, 0]
    for step in sched + [{i: T[i] - sum(x.get(i, 0) for x in sched) for i in range(3)}]:
        ids = [i for i in sorted(step) if step[i] > 0]
        if not ids:
            continue
        log(f"[parity] multi-seq append {[(i, pos[i], step[i]) for i in ids]}")
        kk = np.concatenate([K[i][pos[i]:pos[i] + step[i]] for i in ids])
        vv = np.concatenate([V[i][pos[i]:pos[i] + step[i]] for i in ids])
        ctx.append(0, ids, [step[i] for i in ids], torch.from_numpy(kk.view(np.float16)).to(dev),
                   torch.from_numpy(vv.view(np.float16)).to(dev))
        for i in ids:
            pos[i] += step[i]
    torch.cuda.synchronize()
    assert pos == T
    for i in range(3):
        for g in range(Hkv):
            t1 = orc.build_tier1(np.ascontiguousarray(K[i][:, g]), np.ascontiguousarray(V[i][:, g]))
            compare_tier1(ctx, t1, 0, i, g, f"seq {i} kv {g}")
    ctx.close()


def test_channel_sums_absorption_case(env):
    """Keys constant per channel (1024 on channel 0, 2^-15 elsewhere) and
    q = 1: the ascending fma chains absorb every later term, so every INT8
    score equals fl32(C * 1024) exactly (see the oracle's pin); the whole
    step is compared with the oracle."""
    kvq, torch, orc = env
    d, T, Hkv, Hq = 128, 200, 2, 8
    k = np.full((T, Hkv, d), 2.0 ** -15, np.float32)
    k[:, :, 0] = 1024.0
    v = np.random.default_rng(5).standard_normal((T, Hkv, d)).astype(np.float32)
    q = np.ones((Hq, d), np.float32)
    case = Case("absorption", Hq, Hkv, d, [(S.to16(k), S.to16(v), S.to16(q), None)])
    gpu, ref = _check(env, case)
    C = np.float32(orc.lib().orc_query_scale(d))
    want = (np.float32(C) * np.float32(1024.0)).view(np.uint32)
    assert np.all(f32bits(gpu["trace"][0]["shat"]) == want)
    gpu["ctx"].close()


def test_tier1_d64_and_config1(env):
    kvq, torch, orc = env
    w = S.workload(1)
    case = _wl_case(w, [0])
    gpu = run_gpu(kvq, torch, case, chunks=[100, 1, 1, 600])
    K, V = case.seqs[0][0], case.seqs[0][1]
    t1 = orc.build_tier1(np.ascontiguousarray(K[:, 0]), np.ascontiguousarray(V[:, 0]))
    compare_tier1(gpu["ctx"], t1, 0, 0, 0, "config 1")
    gpu["ctx"].close()


def test_decode_tiny_config1(env):
    gpu, ref = _check(env, _wl_case(S.workload(1), [0]))
    gpu["ctx"].close()


@pytest.mark.parametrize("T,Hq,Hkv,d", [(700, 8, 2, 128), (65, 4, 4, 64), (1, 4, 1, 128),
                                        (130, 8, 4, 128)])
def test_decode_ragged(env, T, Hq, Hkv, d):
    gpu, ref = _check(env, _random_case(f"ragged-{T}-{Hq}q{Hkv}kv-d{d}", T, Hq, Hkv, d, 7))
    gpu["ctx"].close()


def test_decode_llama_layer_8k_with_append(env):
    w = S.workload(2)
    gpu, ref = _check(env, _wl_case(w, [0], extra=True))
    st = gpu["stats"]
    log(f"[parity] 8K stats {st}")
    assert st["promoted_key_blocks"] > 0
    gpu["ctx"].close()


def test_decode_needle_multi_sequence(env):
    w = S.workload(3)
    w.ctx = [4096, 3000]
    w.max_tokens = 4096 + 64
    gpu, ref = _check(env, _wl_case(w, [0, 1], name="needle-2seq"))
    gpu["ctx"].close()


def test_ladder_near_tied_and_rung4(env):
    w = S.workload(5)
    w.ctx = [4096, 2500, 3000]
    w.tied_heads = (2, 8, 0)
    w.hostile_frac = 0.0
    w.max_tokens = 4096 + 64
    gpu, ref = _check(env, _wl_case(w, [0, 1, 2], name="near-tied"))
    assert (gpu["level"][0] == 3).sum() == 8 and np.all(gpu["level"][1] == 4)
    gpu["ctx"].close()


def test_ladder_hostile_values(env):
    w = S.workload(5)
    w.ctx = [3000]
    w.tied_heads = (0,)
    w.max_tokens = 3000 + 64
    gpu, ref = _check(env, _wl_case(w, [0], name="hostile-values"))
    assert np.all(gpu["level"][0] == 2)
    assert gpu["stats"]["promoted_value_blocks"] > 0
    gpu["ctx"].close()


def test_ladder_widening(env):
    case = _random_case("widen", 1500, 4, 1, 64, 103, qscale=3.0, tau_cov_ppm=500_000,
                        eps_key=1e-12, v_tol=1e9)
    gpu, ref = _check(env, case)
    assert np.all(gpu["level"][0] >= 1)
    gpu["ctx"].close()
    case = _random_case("widen-stop", 1500, 4, 1, 64, 103, qscale=3.0, tau_cov_ppm=500_000,
                        eps_key=2e-2, v_tol=1e9)
    gpu, ref = _check(env, case)
    gpu["ctx"].close()


def test_forced_dense_and_full_coverage(env):
    w = S.workload(1)
    gpu, ref = _check(env, _wl_case(w, [0], name="force-dense", force_dense=True))
    assert np.all(gpu["level"] == 4)
    gpu["ctx"].close()
    gpu, ref = _check(env, _wl_case(w, [0], name="tau1-vtol0", tau_cov_ppm=1_000_000, v_tol=0.0))
    gpu["ctx"].close()


def test_deterministic_rerun(env):
    kvq, torch, orc = env
    case = _random_case("rerun", 3000, 8, 2, 128, 9)
    a = run_gpu(kvq, torch, case)
    b = run_gpu(kvq, torch, case)
    for k in ("out", "e_key", "e_val", "level"):
        assert np.array_equal(a[k], b[k]), k
    a["ctx"].close()
    b["ctx"].close()


def test_abi_error_statuses(env):
    kvq, torch, orc = env
    ctx = kvq.Context(2, 2, 8, 2, 128, 100)
    q = torch.zeros((1, 8, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        ctx.decode_step(0, [0], q)
    assert e.value.status == -5                           # empty sequence
    k = torch.zeros((101, 2, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        ctx.append(0, [0], [101], k, k)
    assert e.value.status == -4                           # capacity
    with pytest.raises(kvq.KvqError) as e:
        ctx.append(2, [0], [1], k[:1], k[:1])
    assert e.value.status == -5                           # bad layer
    with pytest.raises(kvq.KvqError) as e:
        ctx.append(0, [0, 0], [1, 1], k[:2], k[:2])
    assert e.value.status == -1                           # duplicate slot
    ctx.append(0, [1], [100], k[:100], k[:100])
    assert ctx.seq_len(0, 1) == 100 and ctx.seq_len(1, 1) == 0
    ctx.reset_seq(1)
    assert ctx.seq_len(0, 1) == 0
    ctx.close()
