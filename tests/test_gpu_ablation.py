"""GPU parity of the FP16-values ablation and a v_tol sweep (needs an MI355X;
marked gpu).

Résultats of the pages: reading values in FP16 closes the accuracy gap that
INT4 values leave; v_tol is the tolerance of rung 2.  Workload: the ladder
stress construction (hostile values in 5 % of the value groups) at 1500
tokens, one sequence, 32 q / 8 KV heads, d 128.

* KVQ_FLAG_FP16_VALUES: every trace (V_g = all blocks, no V_h, E_val = 0,
  no level 2) bit-identical to the oracle, output within 2e-3;
* v_tol in {0, 0.05, 0.25, 1, 1e9}: bit-identical decisions at every value,
  the number of heads at level 2 never grows with v_tol, and every head at
  levels 0-2 meets E_val <= v_tol.
"""
import numpy as np
import pytest

import kvq_synth as S
from gpu_helpers import Case, compare, log, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env(orc):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import certified_quantized_kv_amd as kvq
    return kvq, torch, orc


def _hostile_case(name, **cfg):
    w = S.workload(5)
    w.ctx, w.tied_heads, w.max_tokens = [1500], (0,), 1500 + 64
    K, V = S.prefill(w, 0, 0)
    return Case(name, w.Hq, w.Hkv, w.d, [(K, V, S.query(w, 0, 0, 0), None)],
                max_tokens=w.max_tokens, **cfg)


def _check(env, case):
    kvq, torch, orc = env
    log(f"[ablation] {case.name}: GPU")
    gpu = run_gpu(kvq, torch, case)
    log(f"[ablation] {case.name}: oracle")
    ref = run_oracle(orc, case)
    compare(case, gpu, ref)
    gpu["ctx"].close()
    return gpu, ref


def test_fp16_values_ablation(env):
    gpu, ref = _check(env, _hostile_case("fp16-values", fp16_values=True))
    assert not np.any(gpu["level"] == 2)
    assert np.all(gpu["e_val"] == 0)
    assert np.all(gpu["trace"][0]["V"] == 1)
    assert gpu["stats"]["promoted_value_blocks"] == 8 * ((1500 + 63) // 64)


def test_v_tol_sweep(env):
    counts = []
    for v_tol in (0.0, 0.05, 0.25, 1.0, 1e9):
        gpu, ref = _check(env, _hostile_case(f"v_tol={v_tol}", v_tol=v_tol))
        lv, ev = gpu["level"][0], gpu["e_val"][0]
        ok = lv <= 2
        assert np.all(ev[ok] <= np.float32(v_tol) * (1 + 1e-6) + 0.0)
        counts.append(int((lv == 2).sum()))
        log(f"[ablation] v_tol={v_tol}: level-2 heads {counts[-1]}, "
            f"value blocks {gpu['stats']['promoted_value_blocks']}")
    assert all(a >= b for a, b in zip(counts, counts[1:]))
    assert counts[0] > 0 and counts[-1] == 0
