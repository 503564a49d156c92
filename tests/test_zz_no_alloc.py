"""GPU test of kvq_dense_decode_noalloc, the dense decode entry point that
allocates nothing (its split-K partials live in the library's fixed
per-device scratch array).  Called through the C ABI and compared with the
existing entry point kvq_dense_decode (same kernels, partials in a context's
scratch): bit-identical outputs, on two calls in a row, the second smaller,
and within 2e-3 of the oracle's dense attention; a call whose partials would
not fit is rejected on the host before any launch.
"""
import ctypes

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


def _inputs(seed, n, Hq, Hkv, d, cap):
    r = np.random.default_rng(seed)
    q = S.to16(r.standard_normal((n, Hq, d)).astype(np.float32))
    k = S.to16((r.standard_normal((n, cap, Hkv, d)) * 2).astype(np.float32))
    v = S.to16(r.standard_normal((n, cap, Hkv, d)).astype(np.float32))
    return q, k, v


def _one(env, seed, lens, Hq, Hkv, d, cap):
    kvq, torch, orc = env
    dev = torch.device("cuda:0")
    n = len(lens)
    q, k, v = _inputs(seed, n, Hq, Hkv, d, cap)
    tq = torch.from_numpy(q.view(np.float16)).to(dev)
    tk = torch.from_numpy(k.view(np.float16)).to(dev)
    tv = torch.from_numpy(v.view(np.float16)).to(dev)
    log(f"[noalloc] lens {lens} Hq {Hq} Hkv {Hkv} d {d} cap {cap}: new entry point")
    got = kvq.dense_decode_noalloc(lens, tq, tk, tv)
    torch.cuda.synchronize()
    log("[noalloc] existing entry point")
    ctx = kvq.Context(1, n, Hq, Hkv, d, cap)
    ref = ctx.dense_decode(lens, tq, tk, tv)
    torch.cuda.synchronize()
    ctx.close()
    got, ref = got.cpu().numpy(), ref.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    G = Hq // Hkv
    for i, T in enumerate(lens):
        for g in (0, Hkv - 1):
            o = orc.dense_attention(q[i, g * G:(g + 1) * G], np.ascontiguousarray(k[i, :T, g]),
                                    np.ascontiguousarray(v[i, :T, g]))
            err = np.abs(got[i, g * G:(g + 1) * G].astype(np.float64) - o).max()
            assert err <= TOL_OUT, f"seq {i} kv {g}: {err}"


def test_noalloc_matches_dense_decode_twice(env):
    # a larger call, then a smaller one: the second reuses the array the
    # first left behind
    _one(env, 1, [4100, 3000, 1], 32, 8, 128, 4160)
    _one(env, 2, [700], 8, 2, 64, 800)


def test_noalloc_rejects_partials_beyond_the_array(env):
    kvq, torch, orc = env
    lib = kvq._lib
    dummy = torch.zeros(16, dtype=torch.float32, device="cuda:0")
    p = ctypes.c_void_p(dummy.data_ptr())
    # 4 x 131072 tokens, 8 KV heads of d 128: 17.0 MB of partials > 16 MiB;
    # the host rejects the call before any launch reads the pointers
    lens = (ctypes.c_int32 * 4)(*([131072] * 4))
    st = lib.kvq_dense_decode_noalloc(4, 32, 8, 128, 131072, lens, p, p, p, p, None)
    assert st == -4, st
    assert b"scratch" in lib.kvq_last_error(None)
    n_fit = kvq.NOALLOC_SCRATCH_BYTES // (8 * 256 * 4 * 130 * 4)
    assert n_fit == 3
