"""GPU tests of KVQ_FLAG_RESIDENT_KEYS (needs an MI355X; marked gpu).

Keeping the FP16 keys in device memory (written on append) must change
nothing but the host-link traffic: over several steps with appends in
between (which rewrite the open block, so a stale device copy would show up
in the FP16 scores), every decision array and output of the resident
context is bit-identical to the paging context's, and no key block crosses
the host link.  The second case also checks the result against the oracle.
"""
import numpy as np
import pytest

import kvq_synth as S
from gpu_helpers import Case, compare, log, run_oracle, same_traces

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env(orc):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import certified_quantized_kv_amd as kvq
    return kvq, torch, orc


def _steps(kvq, torch, resident, K, V, appends, qs, Hq, Hkv, d, cap):
    dev = torch.device("cuda:0")
    ctx = kvq.Context(1, 1, Hq, Hkv, d, cap, resident_keys=resident)
    ctx.append(0, [0], [K.shape[0]], torch.from_numpy(K.view(np.float16)).to(dev),
               torch.from_numpy(V.view(np.float16)).to(dev))
    res = []
    for (k1, v1), q in zip(appends, qs):
        if k1.shape[0]:
            ctx.append(0, [0], [k1.shape[0]], torch.from_numpy(k1.view(np.float16)).to(dev),
                       torch.from_numpy(v1.view(np.float16)).to(dev))
        out, ek, ev, lv, st = ctx.decode_step(0, [0], torch.from_numpy(q[None].view(np.float16)).to(dev),
                                              stats=True)
        torch.cuda.synchronize()
        res.append(dict(out=out.cpu().numpy(), ek=ek.cpu().numpy(), ev=ev.cpu().numpy(),
                        lv=lv.cpu().numpy(), st=st, T=ctx.seq_len(0, 0),
                        tr={k: ctx.export_trace(k, 0) for k in kvq.TR}))
    ctx.close()
    return res


def test_resident_keys_bit_identical_over_steps(env):
    kvq, torch, orc = env
    r = np.random.default_rng(21)
    Hq, Hkv, d, T = 8, 2, 128, 1000
    K = (r.standard_normal((T, Hkv, d)) * 2).astype(np.float16).view(np.uint16)
    V = r.standard_normal((T, Hkv, d)).astype(np.float16).view(np.uint16)
    # step 0: no append; then 1, 30 (crosses a block boundary), 0, 64 tokens
    sizes = [0, 1, 30, 0, 64]
    appends = [((r.standard_normal((n, Hkv, d)) * 2).astype(np.float16).view(np.uint16),
                r.standard_normal((n, Hkv, d)).astype(np.float16).view(np.uint16)) for n in sizes]
    qs = [r.standard_normal((Hq, d)).astype(np.float16).view(np.uint16) for _ in sizes]
    cap = T + sum(sizes) + 64
    log("[residency] paging context")
    a = _steps(kvq, torch, False, K, V, appends, qs, Hq, Hkv, d, cap)
    log("[residency] resident context")
    b = _steps(kvq, torch, True, K, V, appends, qs, Hq, Hkv, d, cap)
    for step, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x["out"].view(np.uint32), y["out"].view(np.uint32)), step
        assert np.array_equal(x["lv"], y["lv"]), step
        assert np.array_equal(x["ek"].view(np.uint32), y["ek"].view(np.uint32)), step
        assert np.array_equal(x["ev"].view(np.uint32), y["ev"].view(np.uint32)), step
        same_traces(x["tr"], y["tr"], Hq, Hkv, x["T"], f"step {step}")
        assert x["st"]["promoted_key_blocks"] == y["st"]["promoted_key_blocks"]
    blk = 64 * d * 2
    # resident keys are never copied: only value blocks (rung 2) cross the link
    for step in range(len(sizes)):
        st_a, st_b = a[step]["st"], b[step]["st"]
        assert st_b["h2d_bytes"] == st_b["promoted_value_blocks"] * blk, (step, st_b)
        assert st_b["h2d_bytes"] < st_a["h2d_bytes"]


def test_resident_keys_match_oracle_after_appends(env):
    kvq, torch, orc = env
    w = S.small(cfg_id=93, T=700, Hq=8, Hkv=2, d=128)
    K, V = S.prefill(w, 0, 0)
    ext = S.append_token(w, 0, 0, 0)
    q = S.query(w, 0, 0, 0)
    case = Case("resident-700+1", w.Hq, w.Hkv, w.d, [(K, V, q, ext)], resident_keys=True)
    dev = torch.device("cuda:0")
    ctx = kvq.Context(1, 1, w.Hq, w.Hkv, w.d, case.max_tokens, resident_keys=True)
    ctx.append(0, [0], [K.shape[0]], torch.from_numpy(K.view(np.float16)).to(dev),
               torch.from_numpy(V.view(np.float16)).to(dev))
    qd = torch.from_numpy(q[None].view(np.float16)).to(dev)
    ctx.decode_step(0, [0], qd)              # makes blocks resident, open block included
    ctx.append(0, [0], [1], torch.from_numpy(ext[0].view(np.float16)).to(dev),
               torch.from_numpy(ext[1].view(np.float16)).to(dev))
    out, ek, ev, lv, stats = ctx.decode_step(0, [0], qd, stats=True)
    torch.cuda.synchronize()
    gpu = dict(out=out.cpu().numpy(), e_key=ek.cpu().numpy(), e_val=ev.cpu().numpy(),
               level=lv.cpu().numpy(), stats=stats,
               trace=[{k: ctx.export_trace(k, 0) for k in kvq.TR}], ctx=ctx)
    ref = run_oracle(orc, case)
    compare(case, gpu, ref)
    ctx.close()
