"""The C-ABI library loads and exports every symbol include/kvq.h declares;
host-side validation paths that return before any device call (CPU only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def kvq():
    import certified_quantized_kv_amd as m
    return m


def test_library_exports_every_declared_symbol(kvq):
    lib = ctypes.CDLL(kvq.LIB_PATH)
    names = _declared()
    assert len(names) >= 15
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) == set(kvq.EXPORTED)


def test_tier1_byte_accounting(kvq):
    # INT8 keys d + key meta 4d/64 + INT4 values d/2 + value meta 4d/32 + eta 4/64
    assert kvq.tier1_bytes_per_token(128) == 216.0625
    assert kvq.tier1_bytes_per_token(64) == 108.0625
    assert abs(kvq.tier1_bytes_per_token(128) / 512 - 0.422) < 1e-3


def test_strerror_and_invalid_configs(kvq):
    lib = kvq._lib
    assert lib.kvq_strerror(0) == b"ok"
    assert lib.kvq_strerror(-4) == b"sequence capacity exceeded"
    bad = [
        dict(head_dim=96), dict(n_q_heads=32, n_kv_heads=4), dict(n_q_heads=6, n_kv_heads=4),
        dict(max_tokens=0), dict(max_tokens=64 * 4096 + 1), dict(tau_cov_ppm=0),
        dict(tau_cov_ppm=1_000_001), dict(eps_key=-1.0), dict(widen_rounds=-1),
    ]
    for b in bad:
        cfg = kvq.Config()
        base = dict(n_layers=1, max_batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128,
                    max_tokens=1024)
        base.update({k: v for k, v in b.items() if k in base})
        lib.kvq_default_config(ctypes.byref(cfg), base["n_layers"], base["max_batch"],
                               base["n_q_heads"], base["n_kv_heads"], base["head_dim"],
                               base["max_tokens"])
        for k, v in b.items():
            if k not in base:
                setattr(cfg, k, v)
        out = ctypes.c_void_p()
        assert lib.kvq_create(ctypes.byref(cfg), ctypes.byref(out)) == -1, b
        assert not out.value
    assert lib.kvq_create(None, None) == -1
    assert lib.kvq_append(None, 0, 1, None, None, None, None, None) == -1
    assert lib.kvq_decode_step(None, 0, 1, None, None, None, None, None, None, None, None) == -1
