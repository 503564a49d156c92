#!/usr/bin/env python3
"""Certified decode-attention throughput on a Llama-3.1-8B-shaped KV cache.

Workload (the 128K configuration): batch 1, 32 layers x (32 query / 8 KV
heads, head dim 128), prefill context 131072 tokens of seeded synthetic fp16
K/V (N(0,1), 3 key outlier channels per (layer, KV head) scaled x10, drawn on
the device with torch's seeded generator).  One step = for every layer: append
one new token (quantize-on-append, tier-2 write) and run one certified decode
step (INT8 scoring, top-K* selection, FP16 promotion from pinned host memory,
ranking check and bounds, ladder, split-K decode).  Inputs of the timed steps
(q, k, v) are generated and resident in device memory before timing starts.

value = KV tokens attended per second over the whole job: sum over timed steps
and layers of the context length, divided by the wall time of the timed steps
(which read no per-call statistics back).  step_ms gives the median, 10th and
90th percentile of the per-step times (events on the stream between steps).

Also reported, from the last two steps' queries run again on every layer with
statistics on: per-kernel times stamped by the runtime at each kernel's start
and end on the stream it runs on; the roofline of the dominant kernel; the
quantized-tier pass (INT8 scoring + selection + controller + mixed decode)
against the tier-1 bytes it must read; host-link throughput of promotions.
Then: the dense FP16 (device-resident cache) and naive INT8/INT4 comparators
on the same layers; the CPU oracle timed on four layer-steps (a bounded
sample), whose outputs are also compared with the GPU's for those layers (sampled
parity); the same timed steps on a context that keeps promoted FP16 keys in
device memory across steps; and on one with a device cache of FP16 key blocks
sized so that tier 1 plus the cache take the pages' ~56 % of the dense FP16
cache's device memory; and one layer with every head forced to the dense
fallback (rungs 3/4).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "certified decode-attn KV tokens/s + % HBM peak, Llama-3.1-8B layer at 128K ctx"
HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCES = {
    "k_score_int8": "kvq_score.hip", "k_score_fp16": "kvq_score.hip",
    "k_decode": "kvq_decode.hip", "k_control": "kvq_control.hip", "k_select": "kvq_select.hip",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=8)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--layers", type=int, default=32)
    p.add_argument("--ctx", type=int, default=131072)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-residency", action="store_true",
                   help="skip the second run with promoted FP16 keys kept in device memory")
    p.add_argument("--no-key-cache", action="store_true",
                   help="skip the run with a device cache of FP16 key blocks")
    p.add_argument("--no-comparators", action="store_true",
                   help="skip the dense FP16 (device-resident) and naive INT8/INT4 comparators")
    p.add_argument("--no-dense-fallback", action="store_true",
                   help="skip the one-layer run with every head forced to the dense fallback")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (counter calibration)")
    return p.parse_args()


def calibrate_copy(mib):
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copied {mib} MiB three times")


def source_sha(name):
    path = os.path.join(ROOT, "certified_quantized_kv_amd", "csrc", KERNEL_SOURCES[name])
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def counter_traffic(name, launch_shape):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel source at the same launch shape."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        db = json.load(open(path))
    except ValueError:
        return None
    rec = db.get(name)
    if not rec or rec.get("source_sha") != source_sha(name) or rec.get("shape") != launch_shape:
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (every box here has "
              "one GPU, and this path does not shard across GPUs)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if a.calibrate_copy:
        calibrate_copy(a.calibrate_copy)
        return
    import certified_quantized_kv_amd as kvq
    import kvq_synth as S

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    w = S.workload(4)
    L, Hq, Hkv, d, T0 = a.layers, w.Hq, w.Hkv, w.d, a.ctx
    n_total = a.warmup + a.steps
    max_tokens = T0 + n_total + 1
    t_setup = time.time()
    ctx = kvq.Context(L, 1, Hq, Hkv, d, max_tokens, timing=True)
    log(f"context: device {ctx.device_bytes / 2**30:.2f} GiB, pinned host "
        f"{ctx.host_pinned_bytes / 2**30:.2f} GiB ({time.time() - t_setup:.1f} s)")
    gen = torch.Generator(device=dev)
    keep = not a.no_cpu_baseline
    comp = not a.no_comparators
    NCPU = 4                          # layers in the oracle's sample
    host0 = {}
    dense_k, dense_v = [], []          # FP16 caches in device memory (comparator)
    prefill_ms = []                    # bulk append of each layer (main context)

    def prefill(cx, keep_dense, keep_host0):
        nonlocal host0
        for layer in range(L):
            gen.manual_seed(4_000_000 + layer)
            K = torch.randn((T0, Hkv, d), generator=gen, device=dev, dtype=torch.float32)
            for g in range(Hkv):
                ch = torch.from_numpy(S.outlier_channels(w, layer, g)).to(dev)
                K[:, g, ch] *= w.outlier_scale
            V = torch.randn((T0, Hkv, d), generator=gen, device=dev, dtype=torch.float32)
            K, V = K.half(), V.half()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            cx.append(layer, [0], [T0], K, V)
            e1.record()
            if cx is ctx:
                e1.synchronize()
                prefill_ms.append(e0.elapsed_time(e1))
            if keep_dense:
                kd = torch.zeros((1, max_tokens, Hkv, d), dtype=torch.float16, device=dev)
                vd = torch.zeros_like(kd)
                kd[0, :T0] = K
                vd[0, :T0] = V
                dense_k.append(kd)
                dense_v.append(vd)
            if keep_host0 and layer < NCPU:
                host0[layer] = (K.cpu().numpy().view(np.uint16), V.cpu().numpy().view(np.uint16))
            del K, V

    prefill(ctx, comp, keep)
    # inputs of every step, resident before timing
    qs, k1s, v1s = [], [], []
    for s in range(n_total):
        gen.manual_seed(5_000_000 + s)
        qs.append(torch.randn((L, 1, Hq, d), generator=gen, device=dev).half())
        k = torch.randn((L, 1, Hkv, d), generator=gen, device=dev)
        for layer in range(L):
            for g in range(Hkv):
                ch = torch.from_numpy(S.outlier_channels(w, layer, g)).to(dev)
                k[layer, :, g, ch] *= w.outlier_scale
        k1s.append(k.half())
        v1s.append(torch.randn((L, 1, Hkv, d), generator=gen, device=dev).half())
    out = torch.empty((1, Hq, d), dtype=torch.float32, device=dev)
    ek = torch.empty((1, Hq), dtype=torch.float32, device=dev)
    ev = torch.empty((1, Hq), dtype=torch.float32, device=dev)
    lv = torch.empty((1, Hq), dtype=torch.int8, device=dev)
    torch.cuda.synchronize()
    log(f"prefill {L} layers x {T0} tokens done ({time.time() - t_setup:.1f} s)")

    recs = []
    step_ms = []

    def run_steps(cx):
        """Warm-up, then the timed steps (append + certified decode per layer,
        no per-call stats readback); returns (wall seconds, KV tokens).  An
        event on the stream after each timed step gives the per-step times
        (no extra synchronisation)."""
        toks = [0]

        def step(s, timed):
            # after this step's append every layer holds T0 + s + 1 tokens
            # (checked against the library once the steps are done)
            for layer in range(L):
                cx.append(layer, [0], [1], k1s[s][layer], v1s[s][layer])
                cx.decode_step(layer, [0], qs[s][layer], out, ek, ev, lv, stats=False)
            if timed:
                toks[0] += L * (T0 + s + 1)
        for s in range(a.warmup):
            step(s, False)
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
        t0 = time.time()
        evs[0].record()
        for s in range(a.warmup, n_total):
            step(s, True)
            evs[s - a.warmup + 1].record()
            log(f"step {s - a.warmup + 1}/{a.steps} done")
        torch.cuda.synchronize()
        wall_s = time.time() - t0
        assert all(cx.seq_len(layer, 0) == T0 + n_total for layer in range(L))
        step_ms[:] = [evs[k].elapsed_time(evs[k + 1]) for k in range(a.steps)]
        return wall_s, toks[0]

    def instrument(cx, rec):
        """Per-kernel times, promotions and levels: the last two timed steps'
        queries again on every layer (same shapes), with stats."""
        for s in range(max(a.warmup, n_total - 2), n_total):
            for layer in range(L):
                _, _, _, _, st = cx.decode_step(layer, [0], qs[s][layer], out, ek, ev, lv,
                                                stats=True)
                st["T"] = cx.seq_len(layer, 0)
                rec.append(st)

    def comparators(T_final):
        """Dense FP16 attention over a device-resident cache and the naive
        INT8/INT4 pass over tier 1, on the same layers, lengths and queries
        as the timed certified steps (one untimed warm pass each)."""
        for layer in range(L):
            for s in range(n_total):
                dense_k[layer][0, T0 + s] = k1s[s][layer][0]
                dense_v[layer][0, T0 + s] = v1s[s][layer][0]
        o_d = torch.empty((1, Hq, d), dtype=torch.float32, device=dev)
        res = {}
        for name in ("dense", "naive"):
            def run(s):
                for layer in range(L):
                    if name == "dense":
                        ctx.dense_decode([T_final], qs[s][layer], dense_k[layer], dense_v[layer],
                                         out=o_d)
                    else:
                        ctx.decode_naive(layer, [0], qs[s][layer], out=o_d)
            run(0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for s in range(a.warmup, n_total):
                run(s)
            e1.record()
            e1.synchronize()
            res[name] = e0.elapsed_time(e1) / (a.steps * L)
        dense_bytes = T_final * Hkv * 4 * d
        return {
            "dense_fp16_vram": {
                "what": "dense decode attention, FP16 K/V resident in device memory (same "
                        "layers, lengths and queries)",
                "ms_per_layer": round(res["dense"], 5),
                "kv_tokens_per_s": round(T_final / (res["dense"] * 1e-3), 1),
                "hbm_GBps": round(dense_bytes / (res["dense"] * 1e-3) / 1e9, 1),
                "hbm_frac": round(dense_bytes / (res["dense"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
            "naive_int8_int4": {
                "what": "uncertified INT8 scores + INT4 values over tier 1 (no selection, "
                        "promotion, bounds or ladder)",
                "ms_per_layer": round(res["naive"], 5),
                "kv_tokens_per_s": round(T_final / (res["naive"] * 1e-3), 1)},
        }

    wall, kv_tokens = run_steps(ctx)
    steps_main = sorted(step_ms)
    out_default = out.clone()
    value = kv_tokens / wall
    instrument(ctx, recs)
    n = len(recs)

    def avg(key):
        return sum(r[key] for r in recs) / n

    per_kernel = {k: avg(k) for k in ("ms_score_int8", "ms_select", "ms_score_fp16",
                                      "ms_control", "ms_copy", "ms_decode", "ms_combine",
                                      "ms_dense", "ms_misc", "ms_total")}
    T_avg = sum(r["T"] for r in recs) / n
    t1b = kvq.tier1_bytes_per_token(d)
    bytes_k = T_avg * Hkv * (d + 4 * d / 64)                  # INT8 codes + key meta
    bytes_v = T_avg * Hkv * (d / 2 + 4 * d / 32 + 4 / 64)     # INT4 codes + value meta + eta
    bytes_fp16 = avg("promoted_key_blocks") * 64 * d * 2      # staged FP16 keys read
    cand = {
        "k_score_int8": (per_kernel["ms_score_int8"], bytes_k),
        "k_decode": (per_kernel["ms_decode"], bytes_v),
        "k_score_fp16": (per_kernel["ms_score_fp16"], bytes_fp16),
    }
    dom = max(cand, key=lambda k: cand[k][0])
    ms_dom, by_dom = cand[dom]
    achieved = by_dom / (ms_dom * 1e-3) / 1e9
    shape = f"B1-Hq{Hq}-Hkv{Hkv}-d{d}-T{T0}"
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": counter_traffic(dom, shape), "avg_launch_ms": round(ms_dom, 5),
                "algorithmic_bytes_per_launch": int(by_dom)}
    qp_ms = (per_kernel["ms_score_int8"] + per_kernel["ms_select"] + per_kernel["ms_control"] +
             per_kernel["ms_decode"] + per_kernel["ms_combine"] + per_kernel["ms_misc"])
    qp_bytes = T_avg * Hkv * t1b
    quantized_pass = {
        "ms_per_layer": round(qp_ms, 5), "tier1_bytes_per_layer": int(qp_bytes),
        "GBps": round(qp_bytes / (qp_ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(qp_bytes / (qp_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "kv_tokens_per_s_per_layer": round(T_avg / (qp_ms * 1e-3), 1),
        "per_kernel_hbm_frac": {k: round(v[1] / (v[0] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
                                for k, v in cand.items() if v[0] > 0},
    }
    # the same bytes over the two kernels that stream tier 1 (INT8 scoring and
    # the mixed decode), and the time of the latency-bound controller kernels
    st_ms = per_kernel["ms_score_int8"] + per_kernel["ms_decode"]
    quantized_pass["tier1_streaming_kernels"] = {
        "ms_per_layer": round(st_ms, 5),
        "hbm_frac": round(qp_bytes / (st_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    quantized_pass["controller_ms_per_layer"] = round(qp_ms - st_ms, 5)
    promo = {
        "key_blocks_per_layer": round(avg("promoted_key_blocks"), 1),
        "value_blocks_per_layer": round(avg("promoted_value_blocks"), 1),
        "h2d_MB_per_layer": round(avg("h2d_bytes") / 1e6, 2),
        "h2d_GBps": round(avg("h2d_bytes") / (per_kernel["ms_copy"] * 1e-3) / 1e9, 2)
        if per_kernel["ms_copy"] > 0 else None,
        "host_syncs_per_layer": round(avg("host_syncs"), 2),
    }
    levels = [sum(r["level_count"][k] for r in recs) for k in range(5)]

    cpu = None
    comps = None
    if comp:
        T_final = ctx.seq_len(0, 0)
        comps = comparators(T_final)
        cert_ms = wall / a.steps * 1e3 / L
        kern_ms = sum(per_kernel[k] for k in ("ms_score_int8", "ms_select", "ms_score_fp16",
                                             "ms_control", "ms_decode", "ms_combine", "ms_dense",
                                             "ms_misc"))
        dms = comps["dense_fp16_vram"]["ms_per_layer"]
        comps["certified_ms_per_layer"] = round(cert_ms, 5)
        comps["certified_kernels_ms_per_layer"] = round(kern_ms, 5)
        comps["certified_over_dense"] = round(cert_ms / dms, 2)
        comps["certified_kernels_over_dense"] = round(kern_ms / dms, 2)
        comps["naive_over_dense"] = round(comps["naive_int8_int4"]["ms_per_layer"] / dms, 2)
        del dense_k[:], dense_v[:]

    parity = None
    if keep:
        import oracle
        oracle.build()
        # the state of layers 0 .. NCPU-1 after the last timed step,
        # recomputed on the GPU and on the CPU from the same fp16 inputs
        model = ""
        try:
            with open("/proc/cpuinfo") as f:
                model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
        except OSError:
            pass
        t_step = t_tier1 = 0.0
        toks_cpu = 0
        lv_ok = ek_ok = ev_ok = True
        err = 0.0
        kept = []                      # (q, groups, reference levels) of each sampled layer
        for layer in range(NCPU):
            K0, V0 = host0[layer]
            ks = np.concatenate([K0] + [k1s[s][layer].cpu().numpy().view(np.uint16)
                                        for s in range(n_total)])
            vs = np.concatenate([V0] + [v1s[s][layer].cpu().numpy().view(np.uint16)
                                        for s in range(n_total)])
            q_last = qs[n_total - 1][layer]
            o_gpu, ek_g, ev_g, lv_g, _ = ctx.decode_step(layer, [0], q_last, stats=False)
            torch.cuda.synchronize()
            q16 = q_last[0].cpu().numpy().view(np.uint16)
            tq = time.time()
            groups = []
            for g in range(Hkv):
                k16 = np.ascontiguousarray(ks[:, g])
                v16 = np.ascontiguousarray(vs[:, g])
                groups.append((oracle.build_tier1(k16, v16), k16, v16))
            t_tier1 += time.time() - tq
            tq = time.time()
            ref = oracle.decode_step(oracle.Config(), q16, groups)
            t_step += time.time() - tq
            T_last = ks.shape[0]
            toks_cpu += T_last
            lv_ok &= bool(np.array_equal(lv_g.cpu().numpy()[0], ref.level))
            ek_ok &= bool(np.array_equal(ek_g.cpu().numpy()[0].view(np.uint32), ref.e_key.view(np.uint32)))
            ev_ok &= bool(np.array_equal(ev_g.cpu().numpy()[0].view(np.uint32), ref.e_val.view(np.uint32)))
            err = max(err, float(np.abs(o_gpu.cpu().numpy()[0].astype(np.float64) - ref.out).max()))
            kept.append((q16, groups, ref.level))
            del ks, vs
            log(f"oracle layer {layer} done")
        # the same layer-steps again, one host thread each (the oracle's C
        # routines release the interpreter lock while they run)
        import threading
        par = [None] * NCPU

        def _par(j):
            par[j] = oracle.decode_step(oracle.Config(), kept[j][0], kept[j][1])
        ths = [threading.Thread(target=_par, args=(j,)) for j in range(NCPU)]
        tq = time.time()
        for x in ths:
            x.start()
        for x in ths:
            x.join()
        t_par = time.time() - tq
        par_same = all(np.array_equal(par[j].level, kept[j][2]) for j in range(NCPU))
        del kept, par
        cpu = {"value": round(toks_cpu / t_step, 1), "unit": "KV tokens/s", "cores": 1,
               "kind": "oracle", "host": f"{model}, {os.cpu_count()} logical CPUs visible",
               "sample": f"one certified decode step of each of layers 0-{NCPU - 1} (32 q / 8 KV heads, "
                         f"d 128, {T_last} tokens) after the timed steps; {t_step / NCPU:.2f} s per "
                         f"layer-step, tier-1 quantization {t_tier1 / NCPU:.2f} s per layer (not in value)",
               "threads": {"value": round(toks_cpu / t_par, 1), "cores": NCPU,
                           "how": f"the same {NCPU} layer-steps at once, one host thread each",
                           "levels_equal_to_single_thread": par_same}}
        parity = {"layers": list(range(NCPU)), "tokens": T_last, "levels_equal": lv_ok,
                  "e_key_bits_equal": ek_ok, "e_val_bits_equal": ev_ok,
                  "max_abs_out_err": err, "tol": 2e-3}

    resid = None
    if not a.no_residency:
        # the same steps on a context whose promoted FP16 keys stay in device
        # memory across steps (copied once, again only after an append)
        ctx.close()
        cx2 = kvq.Context(L, 1, Hq, Hkv, d, max_tokens, timing=True, resident_keys=True)
        prefill(cx2, False, False)
        recs2 = []
        wall2, toks2 = run_steps(cx2)
        last2 = out.clone()
        instrument(cx2, recs2)
        n2 = len(recs2)
        dense_bytes = L * max_tokens * Hkv * 4 * d
        resid = {
            "what": "same steps with KVQ_FLAG_RESIDENT_KEYS: FP16 keys kept in device memory "
                    "(written on append), no key page-in",
            "value": round(toks2 / wall2, 1), "unit": "KV tokens/s",
            "ms_per_step": round(wall2 / a.steps * 1e3, 3),
            "h2d_MB_per_layer": round(sum(r["h2d_bytes"] for r in recs2) / n2 / 1e6, 3),
            "ms_copy_per_layer": round(sum(r["ms_copy"] for r in recs2) / n2, 5),
            "device_GiB": round(cx2.device_bytes / 2**30, 2),
            "device_frac_of_dense_fp16_cache": round(cx2.device_bytes / dense_bytes, 3),
            "last_output_bit_equal_to_default": bool(torch.equal(last2, out_default)),
        }
        cx2.close()

    kcache = None
    if not a.no_key_cache:
        # the same steps with a device cache of FP16 key blocks sized so that
        # tier 1 plus the cache take the pages' ~56 % of the dense FP16
        # cache's device memory: (0.56 * 4d - tier-1 bytes) / 2d of the key
        # blocks (27.6 % at d = 128)
        if resid is None:
            ctx.close()
        nbmax = (max_tokens + 63) // 64
        frac = (0.56 * 4 * d - t1b) / (2 * d)
        budget = int(frac * L * Hkv * nbmax)
        cx3 = kvq.Context(L, 1, Hq, Hkv, d, max_tokens, timing=True, key_cache_blocks=budget)
        prefill(cx3, False, False)
        recs3 = []
        wall3, toks3 = run_steps(cx3)
        last3 = out.clone()
        instrument(cx3, recs3)
        n3 = len(recs3)
        dense_bytes = L * max_tokens * Hkv * 4 * d
        cached = sum(r["cached_key_blocks"] for r in recs3)
        paged = sum(r["promoted_key_blocks"] for r in recs3)
        kcache = {
            "what": "same steps with KVQ_FLAG_KEY_CACHE: promoted FP16 key blocks kept in a "
                    "device cache (LRU, blocks used within one pass over the layers are kept)",
            "budget_blocks": budget, "budget_frac_of_key_blocks": round(frac, 4),
            "value": round(toks3 / wall3, 1), "unit": "KV tokens/s",
            "ms_per_step": round(wall3 / a.steps * 1e3, 3),
            "cached_frac_of_promoted": round(cached / max(1, cached + paged), 4),
            "h2d_MB_per_layer": round(sum(r["h2d_bytes"] for r in recs3) / n3 / 1e6, 3),
            "ms_copy_per_layer": round(sum(r["ms_copy"] for r in recs3) / n3, 5),
            "device_GiB": round(cx3.device_bytes / 2**30, 2),
            "device_frac_of_dense_fp16_cache": round(cx3.device_bytes / dense_bytes, 3),
            "last_output_bit_equal_to_default": bool(torch.equal(last3, out_default)),
        }
        cx3.close()

    dense_fb = None
    if not a.no_dense_fallback:
        # rungs 3/4 on one layer of the same shape: every head forced dense,
        # so the step copies the layer's FP16 K and V in and runs the dense
        # kernel on them
        if resid is None and kcache is None:
            ctx.close()
        cx4 = kvq.Context(1, 1, Hq, Hkv, d, max_tokens, timing=True, force_dense=True)
        gen.manual_seed(4_000_000)
        K = torch.randn((T0, Hkv, d), generator=gen, device=dev, dtype=torch.float32)
        for g in range(Hkv):
            ch = torch.from_numpy(S.outlier_channels(w, 0, g)).to(dev)
            K[:, g, ch] *= w.outlier_scale
        V = torch.randn((T0, Hkv, d), generator=gen, device=dev, dtype=torch.float32)
        cx4.append(0, [0], [T0], K.half(), V.half())
        del K, V
        recs4 = []
        for s in range(4):
            st = cx4.decode_step(0, [0], qs[s % n_total][0], out, ek, ev, lv, stats=True)[4]
            if s > 0:
                recs4.append(st)
        torch.cuda.synchronize()
        med = lambda k: float(np.median([r[k] for r in recs4]))
        kb = T0 * Hkv * 4 * d
        dense_fb = {
            "what": "one layer (128K tokens, 8 KV heads) with every head forced to level 4: whole-layer "
                    "FP16 K/V over the host link, dense decode on the staged copy",
            "levels": sorted(set(lv.cpu().numpy().ravel().tolist())),
            "kernel": "k_dense_staged", "ms_kernel": round(med("ms_dense"), 5),
            "algorithmic_bytes": kb, "GBps": round(kb / (med("ms_dense") * 1e-3) / 1e9, 1),
            "hbm_frac": round(kb / (med("ms_dense") * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "ms_copy": round(med("ms_copy"), 4),
            "h2d_GBps": round(med("h2d_bytes") / (med("ms_copy") * 1e-3) / 1e9, 2),
            "ms_step": round(med("ms_total"), 4),
        }
        cx4.close()
        log("dense fallback run done")

    t1_bytes = t1b * T0 * Hkv
    t2_bytes = T0 * Hkv * 4 * d
    pm = float(np.median(prefill_ms))
    append = {
        "what": "quantize-on-append of a layer's 131072-token prefill (tier-1 codes, metadata and "
                "eta written to device memory, FP16 K/V written to pinned host memory through the "
                "device mapping), median over the 32 layers",
        "ms_per_layer": round(pm, 3), "tier1_bytes": int(t1_bytes), "tier2_bytes": int(t2_bytes),
        "tier2_host_GBps": round(t2_bytes / (pm * 1e-3) / 1e9, 2),
        "tier1_GBps": round(t1_bytes / (pm * 1e-3) / 1e9, 1),
    }

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "KV tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(wall / a.steps * 1e3, 3),
        "step_ms": {"median": round(float(np.median(steps_main)), 3),
                    "p10": round(float(np.percentile(steps_main, 10)), 3),
                    "p90": round(float(np.percentile(steps_main, 90)), 3)},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8xi8->i32 scores, u4 values, f32 accumulate", "data": "synthetic",
        "config": {"workload": "llama3.1-8b-shaped 32-layer decode, 128K context, append + "
                               "certified decode per layer per step",
                   "batch": 1, "ctx": T0, "layers": L, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": d, "tau_cov": 0.995},
        "roofline": roofline, "cpu_baseline": cpu,
        "quantized_pass": quantized_pass, "per_kernel_ms": {k: round(v, 5) for k, v in per_kernel.items()},
        "promotion": promo, "level_counts": levels, "comparators": comps, "residency": resid,
        "key_cache": kcache, "dense_fallback": dense_fb, "append": append,
        "parity_sample": parity,
        "tier1_vram_frac_of_fp16": round(t1b / (4 * d), 4),
    }
    print(json.dumps(line), flush=True)
    if resid is None and kcache is None and dense_fb is None:
        ctx.close()


if __name__ == "__main__":
    main()
