"""GPU parity of the two comparators (needs an MI355X; marked gpu).

* kvq_decode_naive: uncertified INT8/INT4 attention over tier 1, against the
  oracle's naive_output (INT8 scores and dequantized INT4 values, fp64);
* kvq_dense_decode: dense FP16 attention over a device-resident cache,
  against the oracle's dense_attention (canonical FP16-key scores, fp64).

Outputs within max-abs 2e-3.  Cases: ragged lengths (not multiples of 64 or
of the 32-token step), one token, several sequences of different lengths in
one call, head dims 64 and 128, GQA groups of 1, 2 and 4, and the
Llama-3.1-8B-shaped layer at 128K context.
"""
import numpy as np
import pytest

import kvq_synth as S
from gpu_helpers import TOL_OUT, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env(orc):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import certified_quantized_kv_amd as kvq
    return kvq, torch, orc


def _seqs(seed, lens, Hq, Hkv, d):
    r = np.random.default_rng(seed)
    out = []
    for T in lens:
        K = (r.standard_normal((T, Hkv, d)) * 1.5).astype(np.float16).view(np.uint16)
        V = r.standard_normal((T, Hkv, d)).astype(np.float16).view(np.uint16)
        q = r.standard_normal((Hq, d)).astype(np.float16).view(np.uint16)
        out.append((K, V, q))
    return out


def _oracle_naive(orc, K, V, q, Hq, Hkv):
    G = Hq // Hkv
    qp = orc.query(q)
    res = []
    for g in range(Hkv):
        t1 = orc.build_tier1(K[:, g, :], V[:, g, :])
        res.append(orc.naive_output(qp[g * G:(g + 1) * G], t1, V[:, g, :]))
    return np.concatenate(res)


def _oracle_dense(orc, K, V, q, Hq, Hkv):
    G = Hq // Hkv
    return np.concatenate([orc.dense_attention(q[g * G:(g + 1) * G], K[:, g, :], V[:, g, :])
                           for g in range(Hkv)])


CASES = [
    ("ragged-8q2kv-d128", 3, [700], 8, 2, 128),
    ("one-token-4q4kv-d64", 4, [1], 4, 4, 64),
    ("batch3-8q4kv-d64", 5, [65, 1000, 130], 8, 4, 64),
    ("batch2-32q8kv-d128", 6, [4097, 2000], 32, 8, 128),
]


@pytest.mark.parametrize("name,seed,lens,Hq,Hkv,d", CASES, ids=[c[0] for c in CASES])
def test_naive_matches_oracle(env, name, seed, lens, Hq, Hkv, d):
    kvq, torch, orc = env
    log(f"[comparators] naive {name}")
    dev = torch.device("cuda:0")
    seqs = _seqs(seed, lens, Hq, Hkv, d)
    ctx = kvq.Context(1, len(lens), Hq, Hkv, d, max(lens) + 64)
    Ks = np.concatenate([s[0] for s in seqs])
    Vs = np.concatenate([s[1] for s in seqs])
    ctx.append(0, list(range(len(lens))), lens, torch.from_numpy(Ks.view(np.float16)).to(dev),
               torch.from_numpy(Vs.view(np.float16)).to(dev))
    q = torch.from_numpy(np.stack([s[2] for s in seqs]).view(np.float16)).to(dev)
    out = ctx.decode_naive(0, list(range(len(lens))), q).cpu().numpy()
    for i, (K, V, qh) in enumerate(seqs):
        ref = _oracle_naive(orc, K, V, qh, Hq, Hkv)
        err = np.abs(out[i] - ref).max()
        assert err < TOL_OUT, (name, i, err)
    # the certified step on the same context still runs and agrees in shape
    o2, _, _, lv, _ = ctx.decode_step(0, list(range(len(lens))), q)
    assert o2.shape == out.shape and int(lv.min()) >= 0
    ctx.close()


@pytest.mark.parametrize("name,seed,lens,Hq,Hkv,d", CASES, ids=[c[0] for c in CASES])
def test_dense_matches_oracle(env, name, seed, lens, Hq, Hkv, d):
    kvq, torch, orc = env
    log(f"[comparators] dense {name}")
    dev = torch.device("cuda:0")
    seqs = _seqs(seed, lens, Hq, Hkv, d)
    cap = max(lens) + 64
    ctx = kvq.Context(1, len(lens), Hq, Hkv, d, cap)
    Kd = np.zeros((len(lens), cap, Hkv, d), np.uint16)
    Vd = np.zeros((len(lens), cap, Hkv, d), np.uint16)
    for i, (K, V, _) in enumerate(seqs):
        Kd[i, :K.shape[0]] = K
        Vd[i, :V.shape[0]] = V
    q = torch.from_numpy(np.stack([s[2] for s in seqs]).view(np.float16)).to(dev)
    out = ctx.dense_decode(lens, q, torch.from_numpy(Kd.view(np.float16)).to(dev),
                           torch.from_numpy(Vd.view(np.float16)).to(dev)).cpu().numpy()
    for i, (K, V, qh) in enumerate(seqs):
        ref = _oracle_dense(orc, K, V, qh, Hq, Hkv)
        err = np.abs(out[i] - ref).max()
        assert err < TOL_OUT, (name, i, err)
    ctx.close()


@pytest.mark.timeout(900)
def test_dense_and_naive_llama_layer_128k(env):
    """The bench's layer shape: 32 q / 8 KV heads, d 128, 131072 + 1 tokens."""
    kvq, torch, orc = env
    dev = torch.device("cuda:0")
    w = S.workload(4)
    log("[comparators] 128K: generating")
    K, V = S.prefill(w, 0, 0)
    k1, v1 = S.append_token(w, 0, 0, 0)
    K = np.concatenate([K, k1])
    V = np.concatenate([V, v1])
    q = S.query(w, 0, 0, 0)
    T = K.shape[0]
    ctx = kvq.Context(1, 1, w.Hq, w.Hkv, w.d, w.max_tokens)
    ctx.append(0, [0], [T], torch.from_numpy(K.view(np.float16)).to(dev),
               torch.from_numpy(V.view(np.float16)).to(dev))
    qd = torch.from_numpy(q[None].view(np.float16)).to(dev)
    Kd = torch.zeros((1, w.max_tokens, w.Hkv, w.d), dtype=torch.float16, device=dev)
    Vd = torch.zeros_like(Kd)
    Kd[0, :T] = torch.from_numpy(K.view(np.float16)).to(dev)
    Vd[0, :T] = torch.from_numpy(V.view(np.float16)).to(dev)
    log("[comparators] 128K: GPU")
    dense = ctx.dense_decode([T], qd, Kd, Vd).cpu().numpy()[0]
    naive = ctx.decode_naive(0, [0], qd).cpu().numpy()[0]
    log("[comparators] 128K: oracle")
    ref_d = _oracle_dense(orc, K, V, q, w.Hq, w.Hkv)
    ref_n = _oracle_naive(orc, K, V, q, w.Hq, w.Hkv)
    ed, en = np.abs(dense - ref_d).max(), np.abs(naive - ref_n).max()
    log(f"[comparators] 128K: dense err {ed:.2e}, naive err {en:.2e}, "
        f"naive vs dense {np.abs(ref_n - ref_d).max():.2e}")
    assert ed < TOL_OUT and en < TOL_OUT
    ctx.close()
