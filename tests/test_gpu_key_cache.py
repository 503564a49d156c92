"""GPU tests of KVQ_FLAG_KEY_CACHE (needs an MI355X; marked gpu).

A device cache of FP16 key blocks must change nothing but where promoted
keys come from: over several steps on two layers, with appends in between
(which change the open block, so a stale cached copy would show up in the
FP16 scores), every decision array and output is bit-identical to the
default context's, cached blocks are counted, and only uncached key blocks
cross the host link.  Every call of the cached context is also compared
with the oracle on that layer's current token stream (tier 2 is the ground
truth every promoted block must reproduce, Méthodologie §1), including the
tiny budget with eviction and bypass, and the refill after kvq_reset_seq.
"""
import numpy as np
import pytest

from gpu_helpers import Case, compare, log, run_oracle, same_traces


def _vs_oracle(orc, Hq, Hkv, d, Kcur, Vcur, q16, res, where):
    """One call of a cached context against the oracle on the layer's token
    stream: every decision array bit for bit, outputs within 2e-3.  Promoted
    blocks counted by the oracle's U_g = host-link blocks + cached blocks."""
    case = Case(where, Hq, Hkv, d, [(Kcur, Vcur, q16, None)])
    st = dict(res["st"])
    st["promoted_key_blocks"] = st["promoted_key_blocks"] + st["cached_key_blocks"]
    gpu = dict(out=res["out"], e_key=res["ek"], e_val=res["ev"], level=res["lv"], stats=st,
               trace=[res["tr"]])
    compare(case, gpu, run_oracle(orc, case))

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env(orc):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import certified_quantized_kv_amd as kvq
    return kvq, torch, orc


def _run(kvq, torch, L, K, V, appends, qs, Hq, Hkv, d, cap, cache_blocks):
    dev = torch.device("cuda:0")
    ctx = kvq.Context(L, 1, Hq, Hkv, d, cap, key_cache_blocks=cache_blocks)
    for layer in range(L):
        ctx.append(layer, [0], [K[layer].shape[0]],
                   torch.from_numpy(K[layer].view(np.float16)).to(dev),
                   torch.from_numpy(V[layer].view(np.float16)).to(dev))
    res = []
    cur = [[K[layer]] for layer in range(L)], [[V[layer]] for layer in range(L)]
    for step, (ap, q) in enumerate(zip(appends, qs)):
        for layer in range(L):
            k1, v1 = ap[layer]
            if k1.shape[0]:
                ctx.append(layer, [0], [k1.shape[0]], torch.from_numpy(k1.view(np.float16)).to(dev),
                           torch.from_numpy(v1.view(np.float16)).to(dev))
                cur[0][layer].append(k1)
                cur[1][layer].append(v1)
            out, ek, ev, lv, st = ctx.decode_step(
                layer, [0], torch.from_numpy(q[layer][None].view(np.float16)).to(dev), stats=True)
            torch.cuda.synchronize()
            res.append(dict(out=out.cpu().numpy(), ek=ek.cpu().numpy(), ev=ev.cpu().numpy(),
                            lv=lv.cpu().numpy(), st=st, T=ctx.seq_len(layer, 0),
                            tr={k: ctx.export_trace(k, 0) for k in kvq.TR},
                            K=np.concatenate(cur[0][layer]), V=np.concatenate(cur[1][layer]),
                            q=q[layer]))
    ctx.close()
    return res


def _case(seed, L, Hq, Hkv, d, T, sizes):
    r = np.random.default_rng(seed)
    K = [(r.standard_normal((T, Hkv, d)) * 2).astype(np.float16).view(np.uint16) for _ in range(L)]
    V = [r.standard_normal((T, Hkv, d)).astype(np.float16).view(np.uint16) for _ in range(L)]
    appends = [[((r.standard_normal((n, Hkv, d)) * 2).astype(np.float16).view(np.uint16),
                 r.standard_normal((n, Hkv, d)).astype(np.float16).view(np.uint16))
                for _ in range(L)] for n in sizes]
    qs = [[r.standard_normal((Hq, d)).astype(np.float16).view(np.uint16) for _ in range(L)]
          for _ in sizes]
    return K, V, appends, qs


# 0.596: the "asymmetric cache configuration" as read here (device memory at
# 72 % of the dense FP16 cache: (0.72 * 4d - 216.06) / 2d of the key blocks)
@pytest.mark.parametrize("frac", [0.4, (0.72 * 512 - 216.0625) / 256, 2.0],
                         ids=["budget-40pct", "budget-asymmetric-59.6pct", "budget-all"])
def test_key_cache_bit_identical_over_steps(env, frac):
    kvq, torch, orc = env
    L, Hq, Hkv, d, T = 2, 8, 2, 128, 1000
    sizes = [0, 1, 30, 0, 64]           # the 30 cross a block boundary
    K, V, appends, qs = _case(31, L, Hq, Hkv, d, T, sizes)
    cap = T + sum(sizes) + 64
    blocks = L * Hkv * ((cap + 63) // 64)
    budget = max(1, int(frac * blocks))
    log(f"[key-cache] default context ({len(sizes)} steps x {L} layers)")
    a = _run(kvq, torch, L, K, V, appends, qs, Hq, Hkv, d, cap, 0)
    log(f"[key-cache] cached context, {budget} slots")
    b = _run(kvq, torch, L, K, V, appends, qs, Hq, Hkv, d, cap, budget)
    blk = 64 * d * 2
    cached_total = 0
    for n, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x["out"].view(np.uint32), y["out"].view(np.uint32)), n
        assert np.array_equal(x["lv"], y["lv"]), n
        assert np.array_equal(x["ek"].view(np.uint32), y["ek"].view(np.uint32)), n
        assert np.array_equal(x["ev"].view(np.uint32), y["ev"].view(np.uint32)), n
        same_traces(x["tr"], y["tr"], Hq, Hkv, x["T"], f"call {n}")
        sa, sb = x["st"], y["st"]
        assert sa["cached_key_blocks"] == 0
        # the same blocks are promoted; the cached ones skip the host link
        assert sb["promoted_key_blocks"] + sb["cached_key_blocks"] == sa["promoted_key_blocks"], n
        assert sb["h2d_bytes"] == sa["h2d_bytes"] - sb["cached_key_blocks"] * blk, n
        if n < L:
            assert sb["cached_key_blocks"] == 0      # first pass over the layers: cache empty
        cached_total += sb["cached_key_blocks"]
        assert y["T"] == y["K"].shape[0]
        _vs_oracle(orc, Hq, Hkv, d, y["K"], y["V"], y["q"], y, f"cached call {n}")
    assert cached_total > 0
    if frac > 1.0:
        # everything fits: after the first pass only blocks changed by an
        # append (or never promoted before) come over the host link
        last = b[-1]["st"]
        assert last["cached_key_blocks"] >= last["promoted_key_blocks"] > 0


def test_key_cache_rejects_residency(env):
    kvq, torch, orc = env
    with pytest.raises(kvq.KvqError):
        kvq.Context(1, 1, 8, 2, 128, 256, resident_keys=True, key_cache_blocks=16)


def test_key_cache_tiny_budget_and_reset(env):
    """Five slots for three layers (constant eviction and bypass), then the
    sequence is reset and refilled with other keys: the cache must serve
    nothing stale, and the results stay bit-identical to the default context."""
    kvq, torch, orc = env
    L, Hq, Hkv, d, T = 3, 8, 2, 128, 500
    sizes = [0, 3, 0, 70]
    cap = 2 * T + sum(sizes) + 64
    dev = torch.device("cuda:0")

    def run(cache_blocks):
        K, V, appends, qs = _case(41, L, Hq, Hkv, d, T, sizes)
        K2, V2, _, _ = _case(42, L, Hq, Hkv, d, T, [0])
        ctx = kvq.Context(L, 1, Hq, Hkv, d, cap, key_cache_blocks=cache_blocks)
        outs = []
        for phase, (KK, VV) in enumerate(((K, V), (K2, V2))):
            if phase == 1:
                ctx.reset_seq(0)
            cur = [[KK[layer]] for layer in range(L)], [[VV[layer]] for layer in range(L)]
            for layer in range(L):
                ctx.append(layer, [0], [KK[layer].shape[0]],
                           torch.from_numpy(KK[layer].view(np.float16)).to(dev),
                           torch.from_numpy(VV[layer].view(np.float16)).to(dev))
            for ap, q in zip(appends, qs):
                for layer in range(L):
                    k1, v1 = ap[layer]
                    if k1.shape[0]:
                        ctx.append(layer, [0], [k1.shape[0]],
                                   torch.from_numpy(k1.view(np.float16)).to(dev),
                                   torch.from_numpy(v1.view(np.float16)).to(dev))
                        cur[0][layer].append(k1)
                        cur[1][layer].append(v1)
                    out, ek, ev, lv, st = ctx.decode_step(
                        layer, [0], torch.from_numpy(q[layer][None].view(np.float16)).to(dev),
                        stats=True)
                    torch.cuda.synchronize()
                    outs.append((out.cpu().numpy(), ek.cpu().numpy(), lv.cpu().numpy(), st,
                                 {k: ctx.export_trace(k, 0) for k in kvq.TR},
                                 ctx.seq_len(layer, 0),
                                 dict(out=out.cpu().numpy(), ek=ek.cpu().numpy(),
                                      ev=ev.cpu().numpy(), lv=lv.cpu().numpy(), st=st,
                                      tr={k: ctx.export_trace(k, 0) for k in kvq.TR}),
                                 np.concatenate(cur[0][layer]), np.concatenate(cur[1][layer]),
                                 q[layer], phase))
        ctx.close()
        return outs

    log("[key-cache] tiny budget: default context")
    a = run(0)
    log("[key-cache] tiny budget: 5 slots")
    b = run(5)
    cached = 0
    for n, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x[0].view(np.uint32), y[0].view(np.uint32)), n
        assert np.array_equal(x[1].view(np.uint32), y[1].view(np.uint32)), n
        assert np.array_equal(x[2], y[2]), n
        same_traces(x[4], y[4], Hq, Hkv, x[5], f"call {n}")
        assert y[3]["promoted_key_blocks"] + y[3]["cached_key_blocks"] == x[3]["promoted_key_blocks"]
        cached += y[3]["cached_key_blocks"]
        assert y[5] == y[7].shape[0]
        _vs_oracle(orc, Hq, Hkv, d, y[7], y[8], y[9], y[6],
                   f"5-slot call {n} ({'after reset' if y[10] else 'before reset'})")
    assert cached > 0
