"""Host-side helpers of the GPU parity tests: run one decode step through the
C ABI and through the oracle on the same inputs, and compare them.

Comparison bar: bit-exact for codes, scales, offsets, eta, INT8/FP16 scores
and every block ingredient, weight, order, selection, verdict, bound and
level; attention outputs within max-abs 2e-3 (fp32 accumulation against the
fp64 oracle); e_key / e_val bit-exact (they are canonical integer ratios),
which is inside the 1e-3 relative bar.
"""
import sys
import numpy as np

TOL_OUT = 2e-3


def f32bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Case:
    """seqs: list of (K, V, q16, extra) with K, V uint16 [T][Hkv][d], q16
    uint16 [Hq][d] and extra = optional (k1, v1) tokens appended in a second
    call before the decode."""

    def __init__(self, name, Hq, Hkv, d, seqs, max_tokens=None, **cfg):
        self.name, self.Hq, self.Hkv, self.d, self.seqs, self.cfg = name, Hq, Hkv, d, seqs, cfg
        T = max(s[0].shape[0] + (0 if s[3] is None else s[3][0].shape[0]) for s in seqs)
        self.max_tokens = max_tokens or (T + 64)


def run_gpu(kvq, torch, case, chunks=None):
    dev = torch.device("cuda:0")
    n = len(case.seqs)
    ctx = kvq.Context(1, n, case.Hq, case.Hkv, case.d, case.max_tokens, **case.cfg)
    if chunks is None:
        Ks = np.concatenate([s[0] for s in case.seqs])
        Vs = np.concatenate([s[1] for s in case.seqs])
        ctx.append(0, list(range(n)), [s[0].shape[0] for s in case.seqs],
                   torch.from_numpy(Ks.view(np.float16)).to(dev),
                   torch.from_numpy(Vs.view(np.float16)).to(dev))
    else:
        for i, (K, V, _, _) in enumerate(case.seqs):
            p = 0
            for c in chunks:
                if p >= K.shape[0]:
                    break
                e = min(K.shape[0], p + c)
                ctx.append(0, [i], [e - p], torch.from_numpy(K[p:e].view(np.float16)).to(dev),
                           torch.from_numpy(V[p:e].view(np.float16)).to(dev))
                p = e
            if p < K.shape[0]:
                ctx.append(0, [i], [K.shape[0] - p], torch.from_numpy(K[p:].view(np.float16)).to(dev),
                           torch.from_numpy(V[p:].view(np.float16)).to(dev))
    ext = [s[3] for s in case.seqs]
    if any(e is not None for e in ext):
        ids = [i for i, e in enumerate(ext) if e is not None]
        k1 = np.concatenate([ext[i][0] for i in ids])
        v1 = np.concatenate([ext[i][1] for i in ids])
        ctx.append(0, ids, [ext[i][0].shape[0] for i in ids],
                   torch.from_numpy(k1.view(np.float16)).to(dev),
                   torch.from_numpy(v1.view(np.float16)).to(dev))
    q = torch.from_numpy(np.stack([s[2] for s in case.seqs]).view(np.float16)).to(dev)
    out, ek, ev, lv, stats = ctx.decode_step(0, list(range(n)), q, stats=True)
    torch.cuda.synchronize()
    res = dict(out=out.cpu().numpy(), e_key=ek.cpu().numpy(), e_val=ev.cpu().numpy(),
               level=lv.cpu().numpy(), stats=stats, trace=[], ctx=ctx)
    for i in range(n):
        res["trace"].append({k: ctx.export_trace(k, i) for k in kvq.TR})
    return res


def full_seq(s):
    K, V, q16, ext = s
    if ext is not None:
        K = np.concatenate([K, ext[0]])
        V = np.concatenate([V, ext[1]])
    return K, V, q16


def run_oracle(orc, case):
    cfgkw = {}
    m = dict(tau_cov_ppm="tau_ppm", eps_key="eps_key", v_tol="v_tol", rho_min_ppm="rho_ppm",
             widen_rounds="widen_rounds", layer_frac_ppm="layer_frac_ppm", force_dense="force_dense",
             fp16_values="fp16_values")
    for k, v in case.cfg.items():
        if k in m:
            cfgkw[m[k]] = v
    cfg = orc.Config(**cfgkw)
    res = []
    for s in case.seqs:
        K, V, q16 = full_seq(s)
        groups = []
        for g in range(case.Hkv):
            k16 = np.ascontiguousarray(K[:, g])
            v16 = np.ascontiguousarray(V[:, g])
            groups.append((orc.build_tier1(k16, v16), k16, v16))
        res.append((orc.decode_step(cfg, q16, groups), groups))
    return res


def same_traces(ta, tb, Hq, Hkv, T, where):
    """Two GPU step traces of the same call are equal everywhere the step
    defines them: FP16 scores and FP16 block ingredients only on promoted
    blocks (elsewhere those arrays keep whatever earlier calls left), INT8
    scores outside them (a step that defers its INT8 scores stores them
    there only)."""
    NB = (T + 63) // 64
    U = ta["U"].reshape(Hkv, NB)
    assert np.array_equal(U, tb["U"].reshape(Hkv, NB)), f"{where}: U"
    G = Hq // Hkv
    Uh = np.repeat(U, G, axis=0) == 1                        # [Hq][NB]
    tokU = Uh[:, np.arange(T) // 64]                         # [Hq][T]
    for k in ta:
        a, b = ta[k], tb[k]
        if k == "sp":
            a, b = a.reshape(Hq, T)[tokU], b.reshape(Hq, T)[tokU]
        elif k == "shat":
            a, b = a.reshape(Hq, T)[~tokU], b.reshape(Hq, T)[~tokU]
        elif k in ("m16", "L16"):
            a, b = a.reshape(Hq, NB)[Uh], b.reshape(Hq, NB)[Uh]
        if a.dtype.kind == "f":
            a, b = a.view(np.uint32 if a.itemsize == 4 else np.uint64), \
                b.view(np.uint32 if b.itemsize == 4 else np.uint64)
        assert np.array_equal(a, b), f"{where}: {k}"


def compare(case, gpu, ref, check_out=True):
    G = case.Hq // case.Hkv
    # every block of every U_g crossed the host link exactly once (the host
    # merges the selection's per-head runs of a group, later rounds add new
    # blocks only)
    nU = sum(int(np.sum(r.groups[g].U)) for r, _ in ref for g in range(case.Hkv))
    # a step that deferred its INT8 scores stored them outside U only
    deferred = bool(gpu["stats"]["scores_deferred"])
    assert gpu["stats"]["promoted_key_blocks"] == nU, \
        f"{case.name}: promoted key blocks {gpu['stats']['promoted_key_blocks']} vs |U| {nU}"
    for i, (r, groups) in enumerate(ref):
        tr_g = gpu["trace"][i]
        T = groups[0][0]["T"]
        NB = (T + 63) // 64
        reshape = lambda a, rows, cols: a.reshape(rows, cols)
        shat = reshape(tr_g["shat"], case.Hq, T)
        sp = reshape(tr_g["sp"], case.Hq, T)
        blk = {k: reshape(tr_g[k], case.Hq, NB) for k in
               ("mhat", "Lhat", "delta", "m16", "L16", "What", "pi", "Wt", "W16", "vh")}
        U = reshape(tr_g["U"], case.Hkv, NB)
        V = reshape(tr_g["V"], case.Hkv, NB)
        for g in range(case.Hkv):
            tr = r.groups[g]
            where = f"{case.name} seq {i} kv {g}"
            assert np.array_equal(U[g], tr.U), f"{where}: U"
            assert np.array_equal(V[g], tr.V), f"{where}: V"
            tokU = tr.U[np.arange(T) // 64] == 1
            for hh in range(G):
                hq = g * G + hh
                w = f"{where} head {hq}"
                sel = ~tokU if deferred else slice(None)
                assert np.array_equal(f32bits(shat[hq][sel]), f32bits(tr.shat[hh][sel])), f"{w}: shat"
                assert np.array_equal(f32bits(blk["delta"][hq]), f32bits(tr.delta[hh])), f"{w}: delta"
                assert np.array_equal(f32bits(blk["mhat"][hq]), f32bits(tr.mhat[hh])), f"{w}: mhat"
                assert np.array_equal(blk["Lhat"][hq], tr.Lhat[hh]), f"{w}: Lhat"
                assert np.array_equal(blk["What"][hq], tr.What[hh]), f"{w}: What"
                assert np.array_equal(blk["pi"][hq], np.array(tr.pi[hh], np.uint32)), f"{w}: pi"
                assert tr_g["k0"][hq] == tr.k0[hh], f"{w}: K*"
                assert tr_g["ssize"][hq] == tr.S_size[hh], f"{w}: |S|"
                assert np.array_equal(f32bits(sp[hq][tokU]), f32bits(tr.sp[hh][tokU])), f"{w}: sp"
                Ub = tr.U == 1
                assert np.array_equal(f32bits(blk["m16"][hq][Ub]), f32bits(tr.m16[hh][Ub])), f"{w}: m16"
                assert np.array_equal(blk["L16"][hq][Ub], tr.L16[hh][Ub]), f"{w}: L16"
                fl = int(tr_g["hflags"][hq])
                assert bool(fl & 1) == tr.consistent[hh], f"{w}: verdict"
                assert bool(fl & 2) == tr.widened[hh], f"{w}: widened"
                assert bool(fl & 4) == tr.failed[hh], f"{w}: rung 3"
                assert (fl >> 8) & 0xff == tr.rounds, f"{w}: rounds"
                assert int(tr_g["ssd"][hq]) == tr.ssd[hh], f"{w}: ssd"
                assert np.array_equal(blk["W16"][hq], tr.W16[hh]), f"{w}: W16"
                assert np.array_equal(blk["Wt"][hq], tr.Wt[hh]), f"{w}: Wt"
                vh = np.zeros(NB, np.uint8)
                vh[tr.V_h[hh]] = 1
                assert np.array_equal(blk["vh"][hq], vh), f"{w}: V_h"
                if not tr.failed[hh]:
                    assert tr_g["ekey64"][hq] == tr.ekey[hh], f"{w}: E_key"
                    assert tr_g["eval64"][hq] == tr.eval[hh], f"{w}: E_val"
        where = f"{case.name} seq {i}"
        assert np.array_equal(gpu["level"][i], r.level), f"{where}: levels {gpu['level'][i]} vs {r.level}"
        assert np.array_equal(f32bits(gpu["e_key"][i]), f32bits(r.e_key)), f"{where}: e_key"
        assert np.array_equal(f32bits(gpu["e_val"][i]), f32bits(r.e_val)), f"{where}: e_val"
        if check_out:
            err = np.abs(gpu["out"][i].astype(np.float64) - r.out).max()
            assert err <= TOL_OUT, f"{where}: max |out - oracle| = {err}"


def compare_tier1(ctx, orc_t1, layer, seq, g, where):
    got = ctx.export_tier1(layer, seq, g)
    for k in ("kcode", "kscale", "koff", "vcode", "vscale", "voff"):
        assert np.array_equal(got[k], orc_t1[k]), f"{where}: {k}"
    for k in ("eta", "vmin", "vmax"):
        assert np.array_equal(f32bits(got[k]), f32bits(orc_t1[k])) or np.array_equal(got[k], orc_t1[k]), \
            f"{where}: {k}"
