"""GPU tests of the ABI boundary (needs an MI355X; marked gpu).

* Canary: a call writes nothing outside the buffers it is given.  Every
  output is a window inside a larger device buffer whose guard regions hold
  a fixed pattern; after the certified step (all four outputs), the naive
  comparator, the dense comparator and the allocation-free dense decode,
  every guard byte is unchanged, and the windows hold what the same calls
  write into plain tensors.
* Launch shapes: the INT8 scoring grid (which wave scores which block, which
  blocks share a batch of channel sums) and the mixed decode's chunk size
  change no decision: every decision array is bit-identical across shapes,
  and the outputs of each shape match the oracle within 2e-3.  With the
  default 48-block chunks the first controller round shares the decode's
  launch (k_eval_decode); 8- and 16-block chunks keep them apart, so both
  routes meet here on the same calls (heads at every rung among them).
"""
import numpy as np
import pytest

import kvq_synth as S
from gpu_helpers import Case, compare, log, run_gpu, run_oracle, same_traces

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes on each side of every output window


@pytest.fixture(scope="module")
def env(orc):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import certified_quantized_kv_amd as kvq
    return kvq, torch, orc


def _guarded(torch, shape, dtype, fill_byte):
    """(window tensor of `shape` inside a byte buffer, the byte buffer)."""
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    buf = torch.full((GUARD + n + GUARD,), fill_byte, dtype=torch.uint8, device="cuda:0")
    win = buf[GUARD:GUARD + n].view(dtype).view(shape)
    return win, buf


def _guards_intact(buf, fill_byte):
    b = buf.cpu().numpy()
    return bool(np.all(b[:GUARD] == fill_byte) and np.all(b[-GUARD:] == fill_byte))


def test_calls_write_only_their_outputs(env):
    kvq, torch, orc = env
    dev = torch.device("cuda:0")
    w = S.small(cfg_id=71, T=1500, Hq=8, Hkv=2, d=128)
    w.ctx = [1500, 1500]
    K, V = S.prefill(w, 0, 0)
    K2, V2 = S.prefill(w, 0, 1)
    n = 2
    q = torch.from_numpy(np.stack([S.query(w, 0, 0, 0), S.query(w, 0, 1, 0)]).view(np.float16)).to(dev)
    ctx = kvq.Context(1, n, w.Hq, w.Hkv, w.d, 1600)
    ctx.append(0, [0, 1], [K.shape[0], K2.shape[0] - 300],
               torch.from_numpy(np.concatenate([K, K2[:-300]]).view(np.float16)).to(dev),
               torch.from_numpy(np.concatenate([V, V2[:-300]]).view(np.float16)).to(dev))
    for fill in (0x5a, 0xff):
        log(f"[boundary] certified step, guard byte {fill:#x}")
        out, bo = _guarded(torch, (n, w.Hq, w.d), torch.float32, fill)
        ek, be = _guarded(torch, (n, w.Hq), torch.float32, fill)
        ev, bv = _guarded(torch, (n, w.Hq), torch.float32, fill)
        lv, bl = _guarded(torch, (n, w.Hq), torch.int8, fill)
        ctx.decode_step(0, [0, 1], q, out, ek, ev, lv)
        torch.cuda.synchronize()
        for b in (bo, be, bv, bl):
            assert _guards_intact(b, fill)
        ref = ctx.decode_step(0, [0, 1], q)
        torch.cuda.synchronize()
        for got, want in zip((out, ek, ev, lv), ref[:4]):
            assert torch.equal(got.cpu(), want.cpu())
        log("[boundary] naive comparator")
        o2, b2 = _guarded(torch, (n, w.Hq, w.d), torch.float32, fill)
        ctx.decode_naive(0, [0, 1], q, out=o2)
        torch.cuda.synchronize()
        assert _guards_intact(b2, fill)
        assert torch.equal(o2.cpu(), ctx.decode_naive(0, [0, 1], q).cpu())
    log("[boundary] dense comparator and the allocation-free dense decode")
    cap = 1600
    kd = torch.zeros((n, cap, w.Hkv, w.d), dtype=torch.float16, device=dev)
    vd = torch.zeros_like(kd)
    kd[0, :K.shape[0]] = torch.from_numpy(K.view(np.float16)).to(dev)
    vd[0, :K.shape[0]] = torch.from_numpy(V.view(np.float16)).to(dev)
    kd[1, :K2.shape[0] - 300] = torch.from_numpy(K2[:-300].view(np.float16)).to(dev)
    vd[1, :K2.shape[0] - 300] = torch.from_numpy(V2[:-300].view(np.float16)).to(dev)
    lens = [K.shape[0], K2.shape[0] - 300]
    o3, b3 = _guarded(torch, (n, w.Hq, w.d), torch.float32, 0x77)
    ctx.dense_decode(lens, q, kd, vd, out=o3)
    o4, b4 = _guarded(torch, (n, w.Hq, w.d), torch.float32, 0x77)
    kvq.dense_decode_noalloc(lens, q, kd, vd, out=o4)
    torch.cuda.synchronize()
    assert _guards_intact(b3, 0x77) and _guards_intact(b4, 0x77)
    assert torch.equal(o3.cpu(), o4.cpu())
    ctx.close()


def test_launch_shapes_do_not_change_decisions(env):
    kvq, torch, orc = env
    w = S.workload(5)
    w.ctx = [4100, 2500, 3000, 700]
    w.tied_heads = (2, 8, 0, 4)
    w.max_tokens = 4160
    rows = []
    for s in range(4):
        K, V = S.prefill(w, 0, s)
        rows.append((K, V, S.query(w, 0, s, 0), None))
    case = Case("launch-shapes", w.Hq, w.Hkv, w.d, rows, max_tokens=w.max_tokens)
    ref = run_oracle(orc, case)
    shapes = [(0, 0), (3, 8), (1, 16), (17, 8), (5, 48)]
    runs = []
    try:
        for sw, mb in shapes:
            kvq.set_launch_shape(sw, mb)
            log(f"[boundary] launch shape: scoring workgroups {sw or 'default'}, "
                f"mixed chunk {mb or 48} blocks")
            g = run_gpu(kvq, torch, case)
            compare(case, g, ref)
            runs.append(g)
    finally:
        kvq.set_launch_shape(0, 0)
    levels = np.concatenate([r.level for r, _ in ref])
    log(f"[boundary] levels {np.bincount(levels, minlength=5).tolist()}")
    a = runs[0]
    for b, (sw, mb) in zip(runs[1:], shapes[1:]):
        for i in range(len(rows)):
            T = rows[i][0].shape[0]
            same_traces(a["trace"][i], b["trace"][i], w.Hq, w.Hkv, T, f"shape {sw}/{mb} seq {i}")
        assert np.array_equal(a["level"], b["level"])
        assert np.array_equal(a["e_key"].view(np.uint32), b["e_key"].view(np.uint32))
        assert np.array_equal(a["e_val"].view(np.uint32), b["e_val"].view(np.uint32))
        b["ctx"].close()
    a["ctx"].close()
