"""The workgroup sort that orders a head's blocks for top-K* selection and for
the ranking check ("Runtime-Certified Bounded-Error Quantized Attention",
Méthodologie §3), called directly through kvq_selftest_sort (needs an MI355X;
marked gpu).

Keys have the blocks' form, weight << 32 | ~block, so they are distinct.  The
result must equal numpy's descending sort of the same unsigned keys, on both
paths of the sort: the bucket sort (spread keys, and keys that tie in their
weight) and its comparison-network fallback, which two tight clusters far
apart force (every key of a cluster lands in one bucket under either bucket
image).  Sizes span one key, one wave, the 1024 threads of the workgroup, and
the largest block count of a sequence (4096), with ragged sizes between.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

SIZES = [1, 2, 63, 64, 65, 1000, 1024, 1025, 2048, 2049, 3001, 4096]


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import certified_quantized_kv_amd as kvq
    return kvq, torch


def _keys(weights):
    n = len(weights)
    b = np.arange(n, dtype=np.uint64)
    return (np.asarray(weights, np.uint64) << np.uint64(32)) | (np.uint64(0xffffffff) - b)


def _run(env, keys):
    kvq, torch = env
    k = torch.from_numpy(keys.view(np.int64).copy()).cuda()
    out, path = kvq.sort_desc(k)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint64)
    want = np.sort(keys)[::-1]
    assert np.array_equal(got, want), f"n={len(keys)}: first mismatch at {np.argmax(got != want)}"
    return int(path.cpu()[0])


@pytest.mark.parametrize("n", SIZES)
def test_sort_spread_weights(env, n):
    r = np.random.default_rng([7, n])
    # block-weight-like: a few heavy blocks, most below 2^31 by a wide range
    w = np.floor(2.0 ** 31 * r.random(n) ** 8).astype(np.uint64)
    _run(env, r.permutation(_keys(w)))


@pytest.mark.parametrize("n", SIZES)
def test_sort_tied_weights(env, n):
    # every block has the same weight: the order is the block index
    keys = _keys(np.full(n, 123456789, np.uint64))
    assert _run(env, np.random.default_rng([8, n]).permutation(keys)) == 0


@pytest.mark.parametrize("n", [100, 1024, 1025, 2048, 2049, 3001, 4096])
def test_sort_clustered_takes_network(env, n):
    r = np.random.default_rng([9, n])
    half = n // 2
    lo = (np.uint64(1) << np.uint64(40)) + r.choice(1 << 20, size=half, replace=False).astype(np.uint64)
    hi = (np.uint64(1) << np.uint64(60)) + r.choice(1 << 20, size=n - half, replace=False).astype(np.uint64)
    keys = r.permutation(np.concatenate([lo, hi]))
    assert _run(env, keys) == 1


def test_sort_rejects_bad_sizes(env):
    kvq, torch = env
    for n in (0, 4097):
        k = torch.ones(max(n, 1), dtype=torch.int64, device="cuda")
        if n == 0:
            k = k[:0]
        with pytest.raises(kvq.KvqError):
            kvq.sort_desc(k)
