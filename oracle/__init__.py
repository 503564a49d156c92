"""CPU oracle of certified quantized-KV decode attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``.  It shares no code with the HIP
product library (certified_quantized_kv_amd) and neither imports the other.

Parity status: every function is pinned by tests/test_oracle_*.py against
properties the page and mathematics fix (round-trip error bound, the score
perturbation bound, E_key >= true TV, E_val >= true value error, the dense
fallback equal to textbook attention and to torch's CPU scaled-dot-product
attention, brute-force selection minimality, a library Spearman).  The
thresholds of the ladder (eps_key, v_tol, rho_min, R1, f_layer) and the 56 %
VRAM figure have no printed value to check against: parity with the page is
unpinned for those numbers, only their validity invariants are pinned.
"""
from ._lib import build, lib
from . import method
from .method import (Config, build_tier1, query, int8_scores, fp16_scores, ingredients,
                     weights, gfactors, attend, value_rows, exp2k, exp2k_coeffs, h2f,
                     rank_order, k_star, ranking_consistent, e_key, e_val_parts, w_bounds,
                     group_step, mixed_output, dense_output, decode_step, f32_up,
                     naive_output, dense_attention, BLOCK, VGROUP)
