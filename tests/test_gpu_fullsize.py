"""GPU parity at the workloads' full sizes (needs an MI355X; marked gpu).

* one Llama-3.1-8B-shaped layer at 128K context plus one appended token, the
  per-layer launch shape of bench.py (batch 1, 32 q / 8 KV heads, d 128);
* four 32K sequences with a planted needle per query head, in one call;
* the adversarial ladder workload: 16 sequences with ragged 4K-64K contexts,
  near-tied key blocks in 0/2/4/8 KV heads per sequence and hostile values in
  5 % of value groups (rungs 2, 3 and 4 all fire).
* the largest context one sequence may hold, 262144 tokens (4096 full blocks
  of 64), on one KV head with its four query heads: the selection and
  controller sorts at their largest size and 256 split-K decode chunks.

Every decision-side array is compared bit for bit with the oracle (scores,
Delta', weights, orders, K*, unions, verdicts, E_key, E_val, V sets, levels)
and every output within max-abs 2e-3.  Level rates of the adversarial
workload are printed.
"""
import numpy as np
import pytest

import kvq_synth as S
from gpu_helpers import Case, compare, log, run_gpu, run_oracle

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


@pytest.fixture(scope="module")
def env(orc):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import certified_quantized_kv_amd as kvq
    return kvq, torch, orc


def _case(w, seqs, name, extra=False, **cfg):
    rows = []
    for s in seqs:
        log(f"[fullsize] {name}: generating sequence {s} ({w.ctx[s]} tokens)")
        K, V = S.prefill(w, 0, s)
        ext = S.append_token(w, 0, s, 0) if extra else None
        rows.append((K, V, S.query(w, 0, s, 0), ext))
    return Case(name, w.Hq, w.Hkv, w.d, rows, max_tokens=w.max_tokens, **cfg)


def _run(env, case):
    kvq, torch, orc = env
    log(f"[fullsize] {case.name}: GPU")
    gpu = run_gpu(kvq, torch, case)
    log(f"[fullsize] {case.name}: oracle")
    ref = run_oracle(orc, case)
    compare(case, gpu, ref)
    lv = gpu["level"]
    log(f"[fullsize] {case.name}: level counts {[int((lv == k).sum()) for k in range(5)]}, "
        f"stats {gpu['stats']}")
    gpu["ctx"].close()
    return gpu


def test_llama_layer_128k_with_append(env):
    w = S.workload(4)
    gpu = _run(env, _case(w, [0], "llama-layer-128k", extra=True))
    assert gpu["stats"]["promoted_key_blocks"] > 0


def test_needle_4x32k(env):
    w = S.workload(3)
    case = _case(w, [0, 1, 2, 3], "needle-4x32k")
    gpu = _run(env, case)
    G = w.Hq // w.Hkv
    first = 0
    for i in range(4):
        pi = gpu["trace"][i]["pi"].reshape(w.Hq, -1)
        ss = gpu["trace"][i]["ssize"]
        for g in range(w.Hkv):
            needles = w.meta["needle_blocks"][(0, i, g)]
            for h in range(G):
                pos = int(np.nonzero(pi[g * G + h] == needles[h])[0][0])
                assert pos < ss[g * G + h]          # the needle is always promoted
                first += pos == 0
    assert first >= 0.9 * 4 * w.Hq                  # and usually the heaviest block


def test_adversarial_ladder_16_sequences(env):
    w = S.workload(5)
    gpu = _run(env, _case(w, list(range(16)), "ladder-16seq"))
    lv = gpu["level"]
    assert (lv == 2).any() and (lv == 3).any() and (lv == 4).any()
    rates = [float((lv == k).mean()) for k in range(5)]
    log(f"[fullsize] ladder level rates {rates}")


def test_max_context_262144_tokens(env):
    w = S.Workload(6, "max-context-256k-4q1kv", 1, 4, 1, 128, [64 * 4096], 3, 10.0,
                   max_tokens=64 * 4096)
    gpu = _run(env, _case(w, [0], w.name))
    tr = gpu["trace"][0]
    assert tr["pi"].size == 4 * 4096
    assert sorted(tr["pi"].reshape(4, -1)[0].tolist()) == list(range(4096))
