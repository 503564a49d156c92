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

roofline = the quantized-tier pass (INT8 scoring, selection, evaluation and
group decisions, mixed decode, combine: every kernel that reads tier 1 plus
the controller between them) against the tier-1 bytes it must read, 216.06 B
per (token, KV head) at d = 128, from per-kernel times stamped by the runtime
at each kernel's start and end, on the last two steps' queries run again on
every layer with statistics on.  dominant_kernel = the kernel with the largest
time of the whole step (the FP16 rescoring of promoted blocks, outside the
pass).

Also reported: the pass at batch 2 and 4 (128K each); the 4 x 32K needle
workload and the 16-sequence adversarial ladder workload (level rates); the
dense FP16 (device-resident) and naive INT8/INT4 comparators; the CPU oracle
on a bounded sample, on one host thread and on every host thread, its
decisions compared with the GPU's for the sampled layers; the same timed
steps with FP16 keys resident in device memory, with a key block cache at the
pages' ~56 % of the dense FP16 cache's memory, and with a key block cache at
72 % (the pages' -28 % "asymmetric cache configuration", as read here); one
layer forced to the dense fallback; the bulk append.

Profiles: `--summarize-profile` turns rocprofv3 output into the summaries kept
under profiles/ (see summarize_profile below).
"""
import argparse
import csv
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "certified decode-attn KV tokens/s + % HBM peak, Llama-3.1-8B layer at 128K ctx"
HBM_PEAK_GBPS = 8000.0
# kernels of the quantized-tier pass and their sources (for counter freshness)
# (every file whose text builds the kernel, past the two common headers)
PASS_KERNELS = {
    "k_score_int8": ("kvq_score.hip",), "k_rescore_int8": ("kvq_score.hip", "kvq_rescore.h"),
    "k_select": ("kvq_select.hip", "kvq_blockops.h"),
    "k_eval": ("kvq_control.hip", "kvq_blockops.h", "kvq_rescore.h"),
    "k_eval_decode": ("kvq_control.hip", "kvq_blockops.h", "kvq_mixed.h", "kvq_rescore.h"),
    "k_decide": ("kvq_control.hip", "kvq_blockops.h"), "k_decode_mixed": ("kvq_decode.hip", "kvq_mixed.h"),
    "k_combine": ("kvq_decode.hip",),
}
OTHER_KERNELS = {"k_score_fp16": ("kvq_score.hip",), "k_dense_vram": ("kvq_dense.hip",),
                 "k_dense_staged": ("kvq_dense.hip",), "k_append": ("kvq_codec.hip",)}
PASS_STATS = ("ms_score_int8", "ms_select", "ms_control", "ms_decode", "ms_combine", "ms_misc")
WORKLOADS = ("batch2_128k", "batch4_128k", "needle_4x32k", "ladder_16seq_4k_64k")


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
                   help="skip the run with promoted FP16 keys kept in device memory")
    p.add_argument("--no-key-cache", action="store_true",
                   help="skip the runs with a device cache of FP16 key blocks (56 %% and 72 %%)")
    p.add_argument("--no-comparators", action="store_true",
                   help="skip the dense FP16 (device-resident) and naive INT8/INT4 comparators")
    p.add_argument("--no-dense-fallback", action="store_true",
                   help="skip the one-layer run with every head forced to the dense fallback")
    p.add_argument("--no-workloads", action="store_true",
                   help="skip the batch-2/4, needle and adversarial-ladder workloads")
    p.add_argument("--only-workload", choices=WORKLOADS, default=None,
                   help="run only this workload and print its record as one JSON line "
                        "(profiling of the batch-2/4 pass, whose decode has a launch of its own "
                        "at batch 4)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (counter calibration)")
    p.add_argument("--summarize-profile", nargs="+", metavar="ARG",
                   help="KIND ARGS...: write a profiles/ summary from rocprofv3 output "
                        "(kinds: kernels, counters, pmc, copies; see summarize_profile)")
    p.add_argument("--cmd", default="", help="the command recorded in a profile summary")
    return p.parse_args()


# ---------------------------------------------------------------------------------
# profile summaries (rocprofv3 output -> profiles/*.txt, profiles/counters.json)
# ---------------------------------------------------------------------------------

def source_sha(name):
    files = (PASS_KERNELS.get(name) or OTHER_KERNELS.get(name)) + ("kvq_device.h", "kvq_internal.h")
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "certified_quantized_kv_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def _short(n):
    n = n.replace("void ", "")
    if "at::" in n:
        return "torch: " + n.split("<")[0][:48]
    return n.split("(")[0][:60]


def _csv(d, name):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(name):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{name} under {d}")


def _dispatch_key(r):
    g = (r.get("Grid_Size_X") or r.get("Grid_Size") or "?", r.get("Grid_Size_Y", ""),
         r.get("Grid_Size_Z", ""))
    return _short(r["Kernel_Name"]), "x".join(x for x in g if x)


def summarize_profile(args, cmd):
    """kernels DIR OUT: per (kernel, grid) dispatch statistics from a
         --kernel-trace run (run_kernel_trace.csv), plus rocprofv3's own
         per-kernel --stats table (run_kernel_stats.csv);
    counters CAL_FETCH CAL_WRITE FETCH WRITE SHAPE OUT_TXT: HBM bytes per
         launch from FETCH_SIZE / WRITE_SIZE runs, scaled by what the same
         counters read for a plain device copy of 1 GiB (bench.py
         --calibrate-copy 1024); writes profiles/counters.json as well;
    pmc DIR OUT: the mean of every collected counter per (kernel, grid);
    copies DIR OUT BENCH_JSON: host-to-device copy durations from a
         --memory-copy-trace run, and GB/s with the bytes from that run's
         bench line."""
    kind = args[0]
    head = [f"# command (run from /tmp on the GPU host, <repo> = repository root):", f"#   {cmd}"]
    if kind == "kernels":
        d, out = args[1], args[2]
        rows = list(csv.DictReader(open(_csv(d, "kernel_trace.csv"))))
        acc = {}
        for r in rows:
            k = _dispatch_key(r)
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            acc.setdefault(k, []).append(dur)
        # grids seen fewer than 3 times (one-off prefills of ragged lengths) and
        # every non-library kernel are pooled per kernel name
        pooled = {}
        for (k, g), v in acc.items():
            key = (k, g) if k.startswith("kvq::") and len(v) >= 3 else (k, "other" if k.startswith("kvq::") else "all")
            pooled.setdefault(key, []).extend(v)
        acc = pooled
        lines = head + ["# per (kernel, grid) over every dispatch of the process; times in microseconds",
                        "#", f"{'kernel':52s} {'grid':>14s} {'calls':>6s} {'avg_us':>9s} {'med_us':>9s} "
                        f"{'min_us':>9s} {'max_us':>9s}"]
        for (k, g), v in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
            v = sorted(v)
            lines.append(f"{k:52s} {g:>14s} {len(v):6d} {sum(v) / len(v):9.2f} {v[len(v) // 2]:9.2f} "
                         f"{v[0]:9.2f} {v[-1]:9.2f}")
        try:
            st = list(csv.DictReader(open(_csv(d, "kernel_stats.csv"))))
            lines += ["#", "# rocprofv3 --stats (per kernel name, all grids):",
                      f"{'kernel':52s} {'calls':>6s} {'avg_us':>9s} {'pct':>7s}"]
            for r in st:
                lines.append(f"{_short(r['Name']):52s} {r['Calls']:>6s} "
                             f"{float(r['AverageNs']) / 1e3:9.2f} {float(r['Percentage']):7.2f}")
        except FileNotFoundError:
            pass
        open(out, "w").write("\n".join(lines) + "\n")
    elif kind == "pmc":
        d, out = args[1], args[2]
        rows = list(csv.DictReader(open(_csv(d, "counter_collection.csv"))))
        acc = {}
        for r in rows:
            k = _dispatch_key(r) + (r["Counter_Name"],)
            if k[0].startswith("kvq::"):        # the library's kernels only
                acc.setdefault(k, []).append(float(r["Counter_Value"]))
        lines = head + ["# mean counter value per dispatch, per (kernel, grid), library kernels", "#"]
        for (k, g, c), v in sorted(acc.items()):
            lines.append(f"{k:52s} {g:>14s} {c:24s} {sum(v) / len(v):16.1f} ({len(v)} dispatches)")
        open(out, "w").write("\n".join(lines) + "\n")
    elif kind == "copies":
        # the trace of this ROCm records no copy sizes: the bytes come from
        # the bench line of the same run (promotion bytes per layer-step x the
        # certified layer-steps it ran: layers x (warmup + steps + 2))
        d, out, bench_json = args[1], args[2], args[3]
        rows = list(csv.DictReader(open(_csv(d, "memory_copy_trace.csv"))))
        acc = {}
        for r in rows:
            direction = r.get("Direction", "?")
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e9
            a = acc.setdefault(direction, [0, 0.0, []])
            a[0] += 1
            a[1] += dur
            a[2].append(dur)
        bl = json.loads(open(bench_json).read().strip().splitlines()[-1])
        steps = bl["config"]["layers"] * (bl["warmup"] + bl["steps"] + 2)
        h2d = bl["promotion"]["h2d_MB_per_layer"] * 1e6 * steps
        lines = head + ["# memory copies by direction: count, summed copy time, median copy time;",
                        f"# host-to-device bytes of the run from its bench line: {steps} certified "
                        f"layer-steps x {bl['promotion']['h2d_MB_per_layer']} MB = {h2d / 1e9:.2f} GB",
                        "#"]
        for k, (n, t, durs) in sorted(acc.items()):
            durs.sort()
            rate = f"{h2d / t / 1e9:8.2f} GB/s" if "HOST_TO_DEVICE" in k and t > 0 else ""
            lines.append(f"{k:28s} {n:7d} copies {t * 1e3:10.2f} ms  median {durs[len(durs) // 2] * 1e6:8.1f} us "
                         f"{rate}")
        open(out, "w").write("\n".join(lines) + "\n")
    elif kind == "counters":
        cf_d, cw_d, f_d, w_d, shape, out = args[1:7]

        def load(d):
            acc = {}
            for r in csv.DictReader(open(_csv(d, "counter_collection.csv"))):
                acc.setdefault(_dispatch_key(r), []).append(float(r["Counter_Value"]))
            return acc
        cf, cw, kf, kw = load(cf_d), load(cw_d), load(f_d), load(w_d)
        copy = [k for k in cf if "copyBuffer" in k[0]][0]
        cal = 1024 * 2 ** 20
        f_fac = cal / (sum(cf[copy]) / len(cf[copy]) * 1024)
        w_fac = cal / (sum(cw[[k for k in cw if "copyBuffer" in k[0]][0]]) /
                       len(cw[[k for k in cw if "copyBuffer" in k[0]][0]]) * 1024)
        # the records of other workload shapes stay; this shape's are replaced
        path = os.path.join(ROOT, "profiles", "counters.json")
        try:
            old = json.load(open(path))
        except (OSError, ValueError):
            old = {}
        db = {name: {key: r for key, r in recs.items() if isinstance(r, dict) and r.get("shape") != shape}
              for name, recs in old.items() if not name.startswith("_") and isinstance(recs, dict)}
        db = {name: recs for name, recs in db.items() if recs}
        cals = {k: v for k, v in old.get("_calibration", {}).items() if isinstance(v, dict)}
        cals[shape] = {"copy_bytes": cal, "fetch_factor": round(f_fac, 4),
                       "write_factor": round(w_fac, 4), "command": cmd}
        db["_calibration"] = cals
        lines = head + [f"# calibration: a plain device copy of {cal} bytes reads FETCH_SIZE "
                        f"{sum(cf[copy]) / len(cf[copy]):.1f} KiB per dispatch: fetched bytes = "
                        f"FETCH_SIZE x 1024 x {f_fac:.4f}, written bytes = WRITE_SIZE x 1024 x {w_fac:.4f}",
                        f"# workload shape {shape}; per (kernel, grid), mean over dispatches", "#"]
        for (k, g), v in sorted(kf.items()):
            full = k.split("::")[-1]
            name = full.split("<")[0]
            if name not in PASS_KERNELS and name not in OTHER_KERNELS:
                continue
            fk = sum(v) / len(v)
            wv = kw.get((k, g))
            if not wv:
                continue
            wk = sum(wv) / len(wv)
            fb, wb = fk * 1024 * f_fac, wk * 1024 * w_fac
            db.setdefault(name, {})[f"{full} {g} {shape}"] = {
                "source_sha": source_sha(name), "shape": shape, "fetch_kib": round(fk, 1),
                "write_kib": round(wk, 1), "hbm_bytes_per_launch": int(fb + wb), "launches": len(v)}
            lines.append(f"{k:40s} grid {g:>12s} FETCH {fk:11.1f} KiB WRITE {wk:10.1f} KiB -> "
                         f"read {fb / 1e6:8.2f} MB + write {wb / 1e6:7.2f} MB = {(fb + wb) / 1e6:8.2f} MB")
        json.dump(db, open(path, "w"), indent=1)
        open(out, "w").write("\n".join(lines) + "\n")
    else:
        raise SystemExit(f"unknown profile summary kind {kind}")
    print(open(out).read())


def counter_traffic(names, shape, optional=()):
    """HBM bytes summed over one launch of each named kernel (its variant and
    grid launched most often at this workload shape: the steady state), from
    the committed counter summary (profiles/counters.json) taken on the
    current kernel sources; None when a kernel of `names` is missing or any
    record used is stale.  Kernels of `optional` count when present."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        db = json.load(open(path))
    except ValueError:
        return None
    tot = 0
    for name in list(names) + list(optional):
        entry = db.get(name, {})
        recs = [r for r in entry.values() if isinstance(r, dict) and r.get("shape") == shape] \
            if isinstance(entry, dict) else []
        if not recs:
            if name in optional:
                continue
            return None
        r = max(recs, key=lambda x: x.get("launches", 0))
        if r.get("source_sha") != source_sha(name):
            return None
        tot += r["hbm_bytes_per_launch"]
    return tot


def calibrate_copy(mib):
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copied {mib} MiB three times")


# ---------------------------------------------------------------------------------
# synthetic inputs on the device (the recipes of kvq_synth, drawn with torch)
# ---------------------------------------------------------------------------------

def pass_summary_of(recs, n_tok_kvh, t1b):
    """Quantized-tier pass from per-call stats: median per kernel class and
    the tier-1 bytes of n_tok_kvh (token, KV head) pairs."""
    import numpy as np
    med = {k: float(np.median([r[k] for r in recs])) for k in
           PASS_STATS + ("ms_score_fp16", "ms_copy", "ms_dense", "ms_total")}
    qp_ms = sum(med[k] for k in PASS_STATS)
    return med, qp_ms, t1b * n_tok_kvh


def gen_kv(torch, gen, dev, w, layer, T, tied=0, hostile=0.0):
    """K, V fp16 [T][Hkv][d]: N(0,1) keys with the layer's outlier channels
    scaled; the first `tied` KV heads repeat one base block in every block plus
    +-0.004 x the channel scale (near-tied block scores); a share `hostile` of
    the (token, 32-channel group) cells of V drawn U(-50, 50)."""
    import kvq_synth as S
    Hkv, d = w.Hkv, w.d
    K = torch.randn((T, Hkv, d), generator=gen, device=dev, dtype=torch.float32)
    for g in range(Hkv):
        ch = torch.from_numpy(S.outlier_channels(w, layer, g)).to(dev)
        scale = torch.ones(d, device=dev)
        scale[ch] = w.outlier_scale
        if g < tied:
            nb = (T + 63) // 64
            base = torch.randn((64, d), generator=gen, device=dev) * scale
            pert = (torch.rand((T, d), generator=gen, device=dev) * 0.008 - 0.004) * scale
            K[:, g, :] = base.repeat(nb, 1)[:T] + pert
        else:
            K[:, g, :] *= scale
    V = torch.randn((T, Hkv, d), generator=gen, device=dev, dtype=torch.float32)
    if hostile > 0:
        ng = d // 32
        Vg = V.view(T, Hkv, ng, 32)
        hit = torch.rand((T, Hkv, ng), generator=gen, device=dev) < hostile
        vals = torch.rand((T, Hkv, ng, 32), generator=gen, device=dev) * 100.0 - 50.0
        Vg[hit] = vals[hit]
    return K.half(), V.half()


def main():
    a = parse()
    if a.summarize_profile:
        summarize_profile(a.summarize_profile, a.cmd)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (the path runs on one "
              "GPU and does not shard across GPUs)", file=sys.stderr)
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
    t1b = kvq.tier1_bytes_per_token(d)
    if a.only_workload:
        res = other_workloads(a, kvq, S, np, torch, torch.Generator(device=dev), dev,
                              lambda recs, n: pass_summary_of(recs, n, t1b), only=a.only_workload)
        print(json.dumps({"workload": a.only_workload, **res[a.only_workload]}), flush=True)
        return
    t_setup = time.time()
    ctx = kvq.Context(L, 1, Hq, Hkv, d, max_tokens, timing=True)
    log(f"context: device {ctx.device_bytes / 2**30:.2f} GiB, pinned host "
        f"{ctx.host_pinned_bytes / 2**30:.2f} GiB ({time.time() - t_setup:.1f} s)")
    gen = torch.Generator(device=dev)
    keep = not a.no_cpu_baseline
    comp = not a.no_comparators
    # layers sampled for the CPU oracle: one per host thread the oracle may use
    n_threads = max(1, min(16, os.cpu_count() or 1))
    NCPU = min(L, max(4, n_threads)) if keep else 0
    host0 = {}
    dense_k, dense_v = [], []          # FP16 caches in device memory (comparator)
    prefill_ms = []                    # bulk append of each layer (main context)

    def prefill(cx, keep_dense, keep_host0):
        for layer in range(L):
            gen.manual_seed(4_000_000 + layer)
            K, V = gen_kv(torch, gen, dev, w, layer, T0)
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
                st = cx.decode_step(layer, [0], qs[s][layer], out, ek, ev, lv, stats=True)[4]
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

    def pass_summary(recs, n_tok_kvh):
        return pass_summary_of(recs, n_tok_kvh, t1b)

    wall, kv_tokens = run_steps(ctx)
    steps_main = sorted(step_ms)
    out_default = out.clone()
    value = kv_tokens / wall
    recs = []
    instrument(ctx, recs)
    n = len(recs)

    def avg(key, rr=recs):
        return sum(r[key] for r in rr) / len(rr)

    per_kernel = {k: avg(k) for k in ("ms_score_int8", "ms_select", "ms_score_fp16",
                                      "ms_control", "ms_copy", "ms_decode", "ms_combine",
                                      "ms_dense", "ms_misc", "ms_total")}
    T_avg = sum(r["T"] for r in recs) / n
    shape = f"B1-Hq{Hq}-Hkv{Hkv}-d{d}-T{T0}"
    qp_ms = sum(per_kernel[k] for k in PASS_STATS)
    qp_bytes = T_avg * Hkv * t1b
    achieved = qp_bytes / (qp_ms * 1e-3) / 1e9
    # the first controller round and the decode share one launch (k_eval_decode)
    # when the call is small enough; its time is then in ms_decode
    fused = per_kernel["ms_control"] == 0.0 and per_kernel["ms_decode"] > 0.0
    pass_names = ["k_score_int8", "k_select", "k_combine"] + (
        ["k_eval_decode"] if fused else ["k_eval", "k_decode_mixed"])
    roofline = {
        "bound": "hbm", "kernel": "quantized-tier pass: k_score_int8 (+ k_rescore_int8 when a step that "
                                  "deferred its INT8 scores and starts with the group pass leaves "
                                  "blocks outside U) + k_select + "
                                  + ("k_eval_decode (first controller round and mixed decode in one launch)"
                                     if fused else "k_eval + k_decode_mixed")
                                  + " (+ k_decide when a head is flagged) + k_combine",
        "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": counter_traffic(pass_names, shape, optional=("k_rescore_int8",)),
        "avg_pass_ms": round(qp_ms, 5), "algorithmic_bytes_per_pass": int(qp_bytes),
        "algorithmic_bytes_per_token_kv_head": round(t1b, 4),
        "per_kernel_ms": {k[3:]: round(per_kernel[k], 5) for k in PASS_STATS},
    }
    bytes_k = T_avg * Hkv * (d + 4 * d / 64)                  # INT8 codes + key meta
    bytes_v = T_avg * Hkv * (d / 2 + 4 * d / 32 + 4 / 64)     # INT4 codes + value meta + eta
    bytes_fp16 = avg("promoted_key_blocks") * 64 * d * 2      # staged FP16 keys read
    cand = {
        "k_score_int8": (per_kernel["ms_score_int8"], bytes_k),
        ("k_eval_decode" if fused else "k_decode_mixed"): (per_kernel["ms_decode"], bytes_v),
        "k_score_fp16": (per_kernel["ms_score_fp16"], bytes_fp16),
    }
    dom = max(cand, key=lambda k: cand[k][0])
    ms_dom, by_dom = cand[dom]
    dominant = {"kernel": dom, "scope": "largest kernel time of the whole step",
                "achieved": round(by_dom / (ms_dom * 1e-3) / 1e9, 1), "unit": "GB/s",
                "frac": round(by_dom / (ms_dom * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "avg_launch_ms": round(ms_dom, 5), "algorithmic_bytes_per_launch": int(by_dom)}
    st_ms = per_kernel["ms_score_int8"] + per_kernel["ms_decode"]
    quantized_pass = {
        "batch1": {"ms_per_layer": round(qp_ms, 5), "tier1_bytes_per_layer": int(qp_bytes),
                   "hbm_frac": round(achieved / HBM_PEAK_GBPS, 4),
                   "kv_tokens_per_s_per_layer": round(T_avg / (qp_ms * 1e-3), 1),
                   "streaming_kernels_ms": round(st_ms, 5),
                   "streaming_kernels_hbm_frac": round(qp_bytes / (st_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                   "controller_ms": round(qp_ms - st_ms, 5),
                   "note": ("the first controller round runs inside the decode launch (k_eval_decode): "
                            "streaming_kernels_ms includes it, controller_ms is selection + combine"
                            if fused else "streaming = k_score_int8 + k_decode_mixed")},
        "per_kernel_hbm_frac": {k: round(v[1] / (v[0] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
                                for k, v in cand.items() if v[0] > 0},
    }
    promo = {
        "key_blocks_per_layer": round(avg("promoted_key_blocks"), 1),
        "value_blocks_per_layer": round(avg("promoted_value_blocks"), 1),
        "h2d_MB_per_layer": round(avg("h2d_bytes") / 1e6, 2),
        "h2d_GBps": round(avg("h2d_bytes") / (per_kernel["ms_copy"] * 1e-3) / 1e9, 2)
        if per_kernel["ms_copy"] > 0 else None,
        "host_syncs_per_layer": round(avg("host_syncs"), 2),
    }
    levels = [sum(r["level_count"][k] for r in recs) for k in range(5)]

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

    cpu, parity = None, None
    if keep:
        cpu, parity = cpu_baseline(a, ctx, qs, k1s, v1s, host0, NCPU, n_threads, n_total,
                                   np, torch)
        host0.clear()

    resid = kcache = asym = None
    ctx.close()
    dense_bytes = L * max_tokens * Hkv * 4 * d
    if not a.no_residency:
        # the same steps on a context whose FP16 keys stay in device memory
        cx2 = kvq.Context(L, 1, Hq, Hkv, d, max_tokens, timing=True, resident_keys=True)
        prefill(cx2, False, False)
        wall2, toks2 = run_steps(cx2)
        last2 = out.clone()
        recs2 = []
        instrument(cx2, recs2)
        resid = {
            "what": "same steps with KVQ_FLAG_RESIDENT_KEYS: FP16 keys kept in device memory "
                    "(written on append), no key page-in",
            "value": round(toks2 / wall2, 1), "unit": "KV tokens/s",
            "ms_per_step": round(wall2 / a.steps * 1e3, 3),
            "h2d_MB_per_layer": round(avg("h2d_bytes", recs2) / 1e6, 3),
            "ms_copy_per_layer": round(avg("ms_copy", recs2), 5),
            "device_GiB": round(cx2.device_bytes / 2**30, 2),
            "device_frac_of_dense_fp16_cache": round(cx2.device_bytes / dense_bytes, 3),
            "last_output_bit_equal_to_default": bool(torch.equal(last2, out_default)),
        }
        cx2.close()

    def cached_run(frac, what):
        nbmax = (max_tokens + 63) // 64
        budget = int(frac * L * Hkv * nbmax)
        cx3 = kvq.Context(L, 1, Hq, Hkv, d, max_tokens, timing=True, key_cache_blocks=budget)
        prefill(cx3, False, False)
        wall3, toks3 = run_steps(cx3)
        last3 = out.clone()
        recs3 = []
        instrument(cx3, recs3)
        cached = sum(r["cached_key_blocks"] for r in recs3)
        paged = sum(r["promoted_key_blocks"] for r in recs3)
        res = {
            "what": what, "budget_blocks": budget, "budget_frac_of_key_blocks": round(frac, 4),
            "value": round(toks3 / wall3, 1), "unit": "KV tokens/s",
            "ms_per_step": round(wall3 / a.steps * 1e3, 3),
            "ms_per_step_over_default": round(wall3 / wall, 3),
            "cached_frac_of_promoted": round(cached / max(1, cached + paged), 4),
            "h2d_MB_per_layer": round(avg("h2d_bytes", recs3) / 1e6, 3),
            "ms_copy_per_layer": round(avg("ms_copy", recs3), 5),
            "device_GiB": round(cx3.device_bytes / 2**30, 2),
            "device_frac_of_dense_fp16_cache": round(cx3.device_bytes / dense_bytes, 3),
            "last_output_bit_equal_to_default": bool(torch.equal(last3, out_default)),
        }
        cx3.close()
        return res

    if not a.no_key_cache:
        # tier 1 plus the cache at the pages' ~56 % of the dense FP16 cache's
        # memory: (0.56 * 4d - tier-1 bytes) / 2d of the key blocks (27.6 %)
        kcache = cached_run((0.56 * 4 * d - t1b) / (2 * d),
                            "same steps with KVQ_FLAG_KEY_CACHE sized so tier 1 plus the cache take "
                            "~56 % of the dense FP16 cache's memory")
        # the "asymmetric cache configuration" as read here: keys and values
        # kept asymmetrically in device memory (part of the keys also in FP16,
        # values only quantized), sized to the pages' -28 % against dense FP16
        # at 128K: (0.72 * 4d - tier-1 bytes) / 2d of the key blocks (59.6 %)
        asym = cached_run((0.72 * 4 * d - t1b) / (2 * d),
                          "asymmetric cache configuration (reading): FP16 key block cache sized so "
                          "device memory is 72 % of the dense FP16 cache (-28 %), values quantized only")
        log("key cache runs done")

    dense_fb = None
    if not a.no_dense_fallback:
        # rungs 3/4 on one layer of the same shape: every head forced dense,
        # so the step copies the layer's FP16 K and V in and runs the dense
        # kernel on them
        cx4 = kvq.Context(1, 1, Hq, Hkv, d, max_tokens, timing=True, force_dense=True)
        gen.manual_seed(4_000_000)
        K, V = gen_kv(torch, gen, dev, w, 0, T0)
        cx4.append(0, [0], [T0], K, V)
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

    workloads = None
    if not a.no_workloads:
        workloads = other_workloads(a, kvq, S, np, torch, gen, dev, pass_summary)
        for B in (2, 4):
            r = workloads.get(f"batch{B}_128k")
            if r:
                quantized_pass[f"batch{B}"] = r["quantized_pass"]

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
        "roofline": roofline, "dominant_kernel": dominant, "cpu_baseline": cpu,
        "quantized_pass": quantized_pass,
        "per_kernel_ms": {k: round(v, 5) for k, v in per_kernel.items()},
        "promotion": promo, "level_counts": levels, "comparators": comps, "residency": resid,
        "key_cache": kcache, "asymmetric_cache": asym, "dense_fallback": dense_fb,
        "workloads": workloads, "append": append, "parity_sample": parity,
        "tier1_vram_frac_of_fp16": round(t1b / (4 * d), 4), "profile_shape": shape,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(a, ctx, qs, k1s, v1s, host0, NCPU, n_threads, n_total, np, torch):
    """The oracle on the state of layers 0 .. NCPU-1 after the timed steps
    (the same fp16 inputs the GPU saw), timed on one host thread (layers
    0-3) and with one host thread per layer-step on every host thread the
    process may use (the oracle unchanged: its C routines release the interpreter
    lock while they run); every sampled layer's levels, bound bits and
    outputs are compared with the GPU's."""
    import threading
    import oracle
    oracle.build()
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    Hkv = ctx.Hkv
    qlast, gpu_res, streams = [], [], []
    for layer in range(NCPU):
        K0, V0 = host0[layer]
        ks = np.concatenate([K0] + [k1s[s][layer].cpu().numpy().view(np.uint16) for s in range(n_total)])
        vs = np.concatenate([V0] + [v1s[s][layer].cpu().numpy().view(np.uint16) for s in range(n_total)])
        q_last = qs[n_total - 1][layer]
        o, e1, e2, l_, _ = ctx.decode_step(layer, [0], q_last, stats=False)
        torch.cuda.synchronize()
        gpu_res.append((o.cpu().numpy()[0], e1.cpu().numpy()[0], e2.cpu().numpy()[0], l_.cpu().numpy()[0]))
        qlast.append(q_last[0].cpu().numpy().view(np.uint16))
        streams.append([(np.ascontiguousarray(ks[:, g]), np.ascontiguousarray(vs[:, g]))
                        for g in range(Hkv)])
        del ks, vs
    T_last = streams[0][0][0].shape[0]
    # tier 1 of every sampled (layer, KV head), built on all threads (not in value)
    groups = [[None] * Hkv for _ in range(NCPU)]
    jobs = [(l, g) for l in range(NCPU) for g in range(Hkv)]
    lock = threading.Lock()

    def build_worker():
        while True:
            with lock:
                if not jobs:
                    return
                l, g = jobs.pop()
            k16, v16 = streams[l][g]
            groups[l][g] = (oracle.build_tier1(k16, v16), k16, v16)
    tq = time.time()
    ths = [threading.Thread(target=build_worker) for _ in range(n_threads)]
    for x in ths:
        x.start()
    for x in ths:
        x.join()
    t_tier1 = time.time() - tq
    log(f"oracle tier 1 of {NCPU} layers built ({t_tier1:.1f} s on {n_threads} threads)")
    # one host thread: layers 0-3 in turn
    n1 = min(4, NCPU)
    tq = time.time()
    for layer in range(n1):
        oracle.decode_step(oracle.Config(), qlast[layer], groups[layer])
    t_one = time.time() - tq
    log(f"oracle single-thread {n1} layer-steps: {t_one:.1f} s")
    # every host thread: one layer-step each, all at once
    refs = [None] * NCPU

    def step_worker(l):
        refs[l] = oracle.decode_step(oracle.Config(), qlast[l], groups[l])
    tq = time.time()
    ths = [threading.Thread(target=step_worker, args=(l,)) for l in range(NCPU)]
    for x in ths:
        x.start()
    for x in ths:
        x.join()
    t_all = time.time() - tq
    log(f"oracle {NCPU} layer-steps on {min(NCPU, n_threads)} threads: {t_all:.1f} s")
    lv_ok = ek_ok = ev_ok = True
    err = 0.0
    for l in range(NCPU):
        o, e1, e2, l_ = gpu_res[l]
        r = refs[l]
        lv_ok &= bool(np.array_equal(l_, r.level))
        ek_ok &= bool(np.array_equal(e1.view(np.uint32), r.e_key.view(np.uint32)))
        ev_ok &= bool(np.array_equal(e2.view(np.uint32), r.e_val.view(np.uint32)))
        err = max(err, float(np.abs(o.astype(np.float64) - r.out).max()))
    cores = min(NCPU, n_threads)
    cpu = {"value": round(NCPU * T_last / t_all, 1), "unit": "KV tokens/s", "cores": cores,
           "kind": "oracle", "host": f"{model}, {os.cpu_count()} logical CPUs visible",
           "sample": f"one certified decode step of each of layers 0-{NCPU - 1} (32 q / 8 KV heads, "
                     f"d 128, {T_last} tokens) after the timed steps, one host thread per layer-step, "
                     f"{cores} at once: {t_all:.2f} s; tier-1 quantization of those layers "
                     f"{t_tier1:.2f} s on {n_threads} threads (not in value)",
           "single_thread": {"value": round(n1 * T_last / t_one, 1), "cores": 1,
                             "sample": f"layers 0-{n1 - 1} in turn, {t_one / n1:.2f} s per layer-step"}}
    parity = {"layers": list(range(NCPU)), "tokens": T_last, "levels_equal": lv_ok,
              "e_key_bits_equal": ek_ok, "e_val_bits_equal": ev_ok, "max_abs_out_err": err,
              "tol": 2e-3}
    return cpu, parity


def other_workloads(a, kvq, S, np, torch, gen, dev, pass_summary, only=None):
    """The quantized-tier pass at batch 2 and 4 (128K each, two layers taken in
    turn so tier 1 does not stay in the 256 MB last-level cache), the 4 x 32K
    needle workload and the 16-sequence adversarial ladder workload (only the
    one named `only`, when given)."""
    res = {}
    w4 = S.workload(4)
    Hq, Hkv, d = w4.Hq, w4.Hkv, w4.d
    t1b = kvq.tier1_bytes_per_token(d)

    def streaming_fracs(med, n_tok):
        # the two streaming kernels against their own algorithmic bytes: INT8
        # codes + key metadata, and INT4 codes + value metadata + eta (the
        # decode's launch also holds the first controller round when
        # ms_control is zero)
        dec = "k_eval_decode" if med["ms_control"] == 0.0 else "k_decode_mixed"
        by = {"k_score_int8": (med["ms_score_int8"], n_tok * Hkv * (d + 4 * d / 64)),
              dec: (med["ms_decode"], n_tok * Hkv * (d / 2 + 4 * d / 32 + 4 / 64))}
        return {k: round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4) for k, (ms, b) in by.items() if ms > 0}

    def pass_traffic(med, lens):
        # HBM bytes of one pass from the committed counters of this shape (a
        # batch of equal 128K contexts), or None where none were taken
        if len(set(lens)) != 1 or lens[0] != 131072:
            return None
        names = ["k_score_int8", "k_select", "k_combine"] + (
            ["k_eval_decode"] if med["ms_control"] == 0.0 else ["k_eval", "k_decode_mixed"])
        return counter_traffic(names, f"B{len(lens)}-Hq{Hq}-Hkv{Hkv}-d{d}-T131072",
                               optional=("k_rescore_int8",))

    def run(name, cx, lens, qfn, steps, layers, extra=None):
        recs = []
        for s in range(steps):
            layer = s % layers
            q = qfn(s, layer)
            o, e1, e2, lvl, st = cx.decode_step(layer, list(range(len(lens))), q, stats=True)
            if s >= layers:               # every layer once untimed first
                recs.append(st)
        torch.cuda.synchronize()
        n_tok = sum(lens)
        med, qp_ms, byt = pass_summary(recs, n_tok * Hkv)
        lv_counts = [sum(r["level_count"][k] for r in recs) for k in range(5)]
        tot = sum(lv_counts)
        r = {"sequences": len(lens), "context_tokens": n_tok,
             "ms_step_median": round(med["ms_total"], 4),
             "kv_tokens_per_s": round(n_tok / (med["ms_total"] * 1e-3), 1),
             "quantized_pass": {"ms": round(qp_ms, 5), "tier1_bytes": int(byt),
                                "hbm_frac": round(byt / (qp_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                                "per_kernel_ms": {k[3:]: round(med[k], 5) for k in PASS_STATS},
                                "per_kernel_hbm_frac": streaming_fracs(med, n_tok),
                                "traffic": pass_traffic(med, lens)},
             "ms_score_fp16": round(med["ms_score_fp16"], 5), "ms_copy": round(med["ms_copy"], 4),
             "ms_dense": round(med["ms_dense"], 5),
             "level_rates": [round(x / tot, 4) for x in lv_counts]}
        if extra:
            r.update(extra(cx))
        res[name] = r
        log(f"workload {name}: {r['ms_step_median']} ms per step, pass frac "
            f"{r['quantized_pass']['hbm_frac']}, levels {r['level_rates']}")

    # batch 2 and 4 at 128K
    for B in (2, 4):
        if only not in (None, f"batch{B}_128k"):
            continue
        T = 131072
        cx = kvq.Context(2, B, Hq, Hkv, d, T + 64, timing=True)
        for layer in range(2):
            for i in range(B):
                gen.manual_seed(6_000_000 + 1000 * B + 10 * layer + i)
                K, V = gen_kv(torch, gen, dev, w4, layer, T)
                cx.append(layer, [i], [T], K, V)
                del K, V
        gen.manual_seed(6_500_000 + B)
        qb = [torch.randn((B, Hq, d), generator=gen, device=dev).half() for _ in range(8)]
        run(f"batch{B}_128k", cx, [T] * B, lambda s, l: qb[s], 8, 2)
        cx.close()

    if only in (None, "needle_4x32k"):
        # 4 x 32K with a planted needle per query head: that head's query
        # direction scaled to 0.8 sqrt(d), plus 0.1 N(0,1), in one block of its KV
        # head (distinct blocks within a KV head)
        w3 = S.workload(3)
        T, B, G = 32768, 4, Hq // Hkv
        cx = kvq.Context(1, B, Hq, Hkv, d, T + 64, timing=True)
        gen.manual_seed(6_700_000)
        q3 = torch.randn((B, Hq, d), generator=gen, device=dev).half()
        needles = {}
        for i in range(B):
            gen.manual_seed(6_710_000 + i)
            K, V = gen_kv(torch, gen, dev, w3, 0, T)
            K = K.float()
            for g in range(Hkv):
                blocks = torch.randperm(T // 64, generator=gen, device=dev)[:G].tolist()
                for hh in range(G):
                    qh = q3[i, g * G + hh].float()
                    b = blocks[hh]
                    K[b * 64:(b + 1) * 64, g, :] = (0.8 * (d ** 0.5) * qh / qh.norm() +
                                                    0.1 * torch.randn((64, d), generator=gen, device=dev))
                    needles[(i, g * G + hh)] = b
            cx.append(0, [i], [T], K.half(), V)
            del K, V

        def needle_check(cx):
            first = 0
            for i in range(B):
                pi = cx.export_trace("pi", i).reshape(Hq, -1)
                first += sum(int(pi[h][0]) == needles[(i, h)] for h in range(Hq))
            return {"needle_ranked_first_frac": round(first / (B * Hq), 4)}
        run("needle_4x32k", cx, [T] * B, lambda s, l: q3, 6, 1, needle_check)
        cx.close()

    if only in (None, "ladder_16seq_4k_64k"):
        # adversarial ladder stress: 16 sequences, contexts 4K-64K, near-tied key
        # blocks in (0, 2, 4, 8)[i mod 4] KV heads of sequence i, 5 % hostile
        # value cells
        w5 = S.workload(5)
        lens = list(w5.ctx)
        cx = kvq.Context(1, len(lens), Hq, Hkv, d, max(lens) + 64, timing=True)
        for i, T in enumerate(lens):
            gen.manual_seed(6_900_000 + i)
            K, V = gen_kv(torch, gen, dev, w5, 0, T, tied=w5.tied_heads[i], hostile=w5.hostile_frac)
            cx.append(0, [i], [T], K, V)
            del K, V
        gen.manual_seed(6_950_000)
        q5 = torch.randn((len(lens), Hq, d), generator=gen, device=dev).half()
        run("ladder_16seq_4k_64k", cx, lens, lambda s, l: q5, 4, 1)
        cx.close()
    return res


if __name__ == "__main__":
    main()
