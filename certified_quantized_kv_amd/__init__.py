"""Python binding of libkvq (certified quantized-KV decode attention on MI355X).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libkvq.so, built in-tree by ``certified_quantized_kv_amd/build.py``.
Importing this package without the built library raises ImportError; there is
no CPU fallback.  PyTorch is used for device memory and streams.

Method: "Runtime-Certified Bounded-Error Quantized Attention" (gist.science
technical summary), Méthodologie §1-§3; see include/kvq.h for the C ABI.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(hipcc --offload-arch=gfx950) first")

_lib = ctypes.CDLL(LIB_PATH)

P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64


class Config(ctypes.Structure):
    _fields_ = [("n_layers", I32), ("max_batch", I32), ("n_q_heads", I32), ("n_kv_heads", I32),
                ("head_dim", I32), ("max_tokens", I32), ("tau_cov_ppm", I32),
                ("rho_min_ppm", I32), ("widen_rounds", I32), ("layer_frac_ppm", I32),
                ("eps_key", ctypes.c_double), ("v_tol", ctypes.c_double),
                ("flags", ctypes.c_uint32), ("key_cache_blocks", I64)]


class StepStats(ctypes.Structure):
    _fields_ = [("promoted_key_blocks", I64), ("promoted_value_blocks", I64),
                ("dense_kv_heads", I64), ("h2d_bytes", I64), ("key_rounds", I32),
                ("host_syncs", I32), ("level_count", I32 * 5),
                ("ms_score_int8", ctypes.c_float), ("ms_select", ctypes.c_float),
                ("ms_score_fp16", ctypes.c_float), ("ms_control", ctypes.c_float),
                ("ms_copy", ctypes.c_float), ("ms_decode", ctypes.c_float),
                ("ms_dense", ctypes.c_float), ("ms_total", ctypes.c_float),
                ("ms_combine", ctypes.c_float), ("ms_misc", ctypes.c_float),
                ("cached_key_blocks", I64), ("scores_deferred", I32)]

    def as_dict(self):
        d = {k: getattr(self, k) for k, _ in self._fields_}
        d["level_count"] = list(self.level_count)
        return d


FLAG_FORCE_DENSE = 1
FLAG_TIMING = 2
FLAG_RESIDENT_KEYS = 4
FLAG_FP16_VALUES = 8
FLAG_KEY_CACHE = 16
FLAG_ALL_SCORES = 32

TR = dict(shat=1, sp=2, mhat=3, Lhat=4, delta=5, m16=6, L16=7, What=8, pi=9, Wt=10, W16=11,
          k0=12, ssize=13, ssd=14, ekey64=15, eval64=16, hflags=17, U=18, V=19, vh=20)
_TR_DTYPE = dict(shat=np.float32, sp=np.float32, mhat=np.float32, Lhat=np.uint32,
                 delta=np.float32, m16=np.float32, L16=np.uint32, What=np.uint32, pi=np.uint32,
                 Wt=np.uint32, W16=np.uint32, k0=np.int32, ssize=np.int32, ssd=np.uint64,
                 ekey64=np.float64, eval64=np.float64, hflags=np.uint32, U=np.uint8, V=np.uint8,
                 vh=np.uint8)

_SIGS = {
    "kvq_default_config": (None, [P, I32, I32, I32, I32, I32, I32]),
    "kvq_create": (I32, [P, P]),
    "kvq_destroy": (None, [P]),
    "kvq_append": (I32, [P, I32, I32, P, P, P, P, P]),
    "kvq_decode_step": (I32, [P, I32, I32, P, P, P, P, P, P, P, P]),
    "kvq_decode_naive": (I32, [P, I32, I32, P, P, P, P]),
    "kvq_dense_decode": (I32, [P, I32, P, P, P, P, P, P]),
    "kvq_reset_seq": (I32, [P, I32]),
    "kvq_seq_len": (I64, [P, I32, I32]),
    "kvq_strerror": (ctypes.c_char_p, [I32]),
    "kvq_last_error": (ctypes.c_char_p, [P]),
    "kvq_tier1_bytes_per_token": (ctypes.c_double, [I32]),
    "kvq_device_bytes": (I64, [P]),
    "kvq_host_pinned_bytes": (I64, [P]),
    "kvq_tier1_export_bytes": (I64, [P, I32, I32]),
    "kvq_export_tier1": (I32, [P, I32, I32, I32, P, ctypes.c_size_t]),
    "kvq_trace_bytes": (I64, [P, I32, I32]),
    "kvq_export_trace": (I32, [P, I32, I32, P, ctypes.c_size_t]),
    "kvq_selftest_exp2k": (I32, [P, P, I64, P]),
    "kvq_selftest_merge_runs": (I32, [P, I64, P, P]),
    "kvq_selftest_sort": (I32, [P, I64, P, P, P]),
    "kvq_dense_decode_noalloc": (I32, [I32, I32, I32, I32, I32, P, P, P, P, P, P]),
    "kvq_selftest_launch_shape": (I32, [I32, I32]),
    "kvq_selftest_defer_scores": (I32, [I32]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class KvqError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"kvq status {status} ({_lib.kvq_strerror(status).decode()}): {msg}")
        self.status = status


def tier1_bytes_per_token(head_dim):
    return _lib.kvq_tier1_bytes_per_token(head_dim)


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _out(t, shape, dtype, device, name):
    """A caller-supplied output: the library writes shape-many elements of
    dtype on device through its pointer, so all three must match exactly."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")
    return _dev(t, dtype, name)


def _i32(seq):
    arr = (I32 * len(seq))(*[int(x) for x in seq])
    return arr


def merge_runs(entries):
    """The host's merge of promotion-plan entries (test hook, no device call):
    entries = sequence of ints len | start << 16 | group << 32 | kind << 48."""
    n = len(entries)
    a = np.ascontiguousarray(np.asarray(entries, dtype=np.uint64))
    out = np.zeros(max(n, 1), np.uint64)
    n_out = ctypes.c_int64(0)
    st = _lib.kvq_selftest_merge_runs(a.ctypes.data_as(P), n, out.ctypes.data_as(P),
                                      ctypes.byref(n_out))
    if st != 0:
        raise KvqError(st, "merge_runs")
    return out[:n_out.value]


def exp2k(x):
    """The library's decision exponential on a float32 CUDA tensor (test hook)."""
    import torch
    y = torch.empty_like(x)
    st = _lib.kvq_selftest_exp2k(_dev(x, torch.float32, "x"), _dev(y, torch.float32, "y"),
                                 x.numel(), _stream())
    if st != 0:
        raise KvqError(st, "exp2k")
    return y


def dense_decode_noalloc(seq_lens, q, k, v, out=None):
    """Dense FP16 decode attention with no device allocation in the library
    (kvq_dense_decode_noalloc): q fp16 [n, Hq, d]; k, v fp16 [n, max_tokens,
    Hkv, d]; out f32 [n, Hq, d] (allocated here by torch when not given).
    Its partials use the library's fixed per-device scratch array."""
    import torch
    n = len(seq_lens)
    if q.dim() != 3 or q.shape[0] != n:
        raise ValueError(f"q shape {tuple(q.shape)} does not match {n} sequences")
    Hq, d = q.shape[1], q.shape[2]
    if k.dim() != 4 or tuple(k.shape) != tuple(v.shape) or k.shape[0] != n or k.shape[3] != d:
        raise ValueError(f"k/v shape {tuple(k.shape)} / {tuple(v.shape)} does not match q")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on one device")
    out = torch.empty((n, Hq, d), dtype=torch.float32, device=q.device) if out is None else out
    st = _lib.kvq_dense_decode_noalloc(n, Hq, k.shape[2], d, k.shape[1], _i32(seq_lens),
                                       _dev(q, torch.float16, "q"), _dev(k, torch.float16, "k"),
                                       _dev(v, torch.float16, "v"),
                                       _out(out, (n, Hq, d), torch.float32, q.device, "out"),
                                       _stream())
    if st != 0:
        raise KvqError(st, f"kvq_dense_decode_noalloc: {_lib.kvq_last_error(None).decode()}")
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20


def set_launch_shape(score_wgs=0, mix_blocks=0):
    """Test hook (kvq_selftest_launch_shape): cap the INT8 scoring grid and
    choose the mixed decode's chunk size for later calls; (0, 0) = defaults."""
    st = _lib.kvq_selftest_launch_shape(int(score_wgs), int(mix_blocks))
    if st != 0:
        raise KvqError(st, "kvq_selftest_launch_shape")


def set_defer_scores(ppm=-1):
    """Test hook (kvq_selftest_defer_scores): the U fraction (ppm) of a
    layer's last step from which a step stores the INT8 scores of the blocks
    outside U only; 0 = every step that reads its unions back, -1 = default."""
    st = _lib.kvq_selftest_defer_scores(int(ppm))
    if st != 0:
        raise KvqError(st, "kvq_selftest_defer_scores")


def sort_desc(keys):
    """The library's workgroup sort of block keys (test hook): keys = int64 CUDA
    tensor of n distinct nonzero keys read as unsigned, 1 <= n <= 4096.
    Returns (the keys in descending unsigned order, int32 CUDA tensor holding 0
    if the bucket sort placed them, 1 if the comparison network sorted them)."""
    import torch
    out = torch.empty_like(keys)
    path = torch.full((1,), -1, dtype=torch.int32, device=keys.device)
    st = _lib.kvq_selftest_sort(_dev(keys, torch.int64, "keys"), keys.numel(),
                                _dev(out, torch.int64, "out"), _dev(path, torch.int32, "path"),
                                _stream())
    if st != 0:
        raise KvqError(st, "sort_desc")
    return out, path


class Context:
    """A tiered quantized KV cache on the current device (kvq_create)."""

    def __init__(self, n_layers, max_batch, n_q_heads, n_kv_heads, head_dim, max_tokens,
                 tau_cov_ppm=995_000, eps_key=1e-3, v_tol=0.25, rho_min_ppm=900_000,
                 widen_rounds=2, layer_frac_ppm=500_000, force_dense=False, timing=False,
                 resident_keys=False, fp16_values=False, key_cache_blocks=0, all_scores=False):
        cfg = Config()
        _lib.kvq_default_config(ctypes.byref(cfg), n_layers, max_batch, n_q_heads, n_kv_heads,
                                head_dim, max_tokens)
        cfg.tau_cov_ppm = tau_cov_ppm
        cfg.eps_key = eps_key
        cfg.v_tol = v_tol
        cfg.rho_min_ppm = rho_min_ppm
        cfg.widen_rounds = widen_rounds
        cfg.layer_frac_ppm = layer_frac_ppm
        cfg.flags = ((FLAG_FORCE_DENSE if force_dense else 0) | (FLAG_TIMING if timing else 0) |
                     (FLAG_RESIDENT_KEYS if resident_keys else 0) |
                     (FLAG_FP16_VALUES if fp16_values else 0) |
                     (FLAG_KEY_CACHE if key_cache_blocks > 0 else 0) |
                     (FLAG_ALL_SCORES if all_scores else 0))
        cfg.key_cache_blocks = key_cache_blocks
        self.cfg = cfg
        self._ctx = ctypes.c_void_p()
        st = _lib.kvq_create(ctypes.byref(cfg), ctypes.byref(self._ctx))
        if st != 0:
            raise KvqError(st, "kvq_create")
        self.Hq, self.Hkv, self.d = n_q_heads, n_kv_heads, head_dim

    def _check(self, st, what):
        if st != 0:
            raise KvqError(st, f"{what}: {_lib.kvq_last_error(self._ctx).decode()}")

    def close(self):
        if self._ctx:
            _lib.kvq_destroy(self._ctx)
            self._ctx = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def device_bytes(self):
        return _lib.kvq_device_bytes(self._ctx)

    @property
    def host_pinned_bytes(self):
        return _lib.kvq_host_pinned_bytes(self._ctx)

    def seq_len(self, layer, seq):
        return _lib.kvq_seq_len(self._ctx, layer, seq)

    def reset_seq(self, seq):
        self._check(_lib.kvq_reset_seq(self._ctx, seq), "kvq_reset_seq")

    def append(self, layer, seq_ids, n_new, k, v):
        """k, v: fp16 CUDA tensors [sum(n_new), n_kv_heads, head_dim]."""
        import torch
        n = len(seq_ids)
        kp = _dev(k, torch.float16, "k")
        vp = _dev(v, torch.float16, "v")
        if k.shape != v.shape or k.dim() != 3 or k.shape[0] != sum(n_new) or \
                k.shape[1] != self.Hkv or k.shape[2] != self.d:
            raise ValueError(f"k/v shape {tuple(k.shape)} does not match the call")
        if k.device != v.device:
            raise ValueError("k and v must be on one device")
        self._check(_lib.kvq_append(self._ctx, layer, n, _i32(seq_ids), _i32(n_new), kp, vp,
                                    _stream()), "kvq_append")

    def decode_step(self, layer, seq_ids, q, out=None, e_key=None, e_val=None, level=None,
                    stats=False):
        """q: fp16 CUDA tensor [n, n_q_heads, head_dim].  Returns
        (out f32 [n,Hq,d], e_key f32 [n,Hq], e_val f32 [n,Hq], level int8 [n,Hq], stats)."""
        import torch
        n = len(seq_ids)
        if q.shape != (n, self.Hq, self.d):
            raise ValueError(f"q shape {tuple(q.shape)} != {(n, self.Hq, self.d)}")
        dev = q.device
        out = torch.empty((n, self.Hq, self.d), dtype=torch.float32, device=dev) if out is None else out
        e_key = torch.empty((n, self.Hq), dtype=torch.float32, device=dev) if e_key is None else e_key
        e_val = torch.empty((n, self.Hq), dtype=torch.float32, device=dev) if e_val is None else e_val
        level = torch.empty((n, self.Hq), dtype=torch.int8, device=dev) if level is None else level
        ss = StepStats() if stats else None
        st = _lib.kvq_decode_step(self._ctx, layer, n, _i32(seq_ids), _dev(q, torch.float16, "q"),
                                  _out(out, (n, self.Hq, self.d), torch.float32, dev, "out"),
                                  _out(e_key, (n, self.Hq), torch.float32, dev, "e_key"),
                                  _out(e_val, (n, self.Hq), torch.float32, dev, "e_val"),
                                  _out(level, (n, self.Hq), torch.int8, dev, "level"),
                                  ctypes.byref(ss) if ss is not None else None, _stream())
        self._check(st, "kvq_decode_step")
        return out, e_key, e_val, level, (ss.as_dict() if ss is not None else None)

    def decode_naive(self, layer, seq_ids, q, out=None):
        """Uncertified INT8/INT4 attention over tier 1 (comparator); returns out f32."""
        import torch
        n = len(seq_ids)
        if q.shape != (n, self.Hq, self.d):
            raise ValueError(f"q shape {tuple(q.shape)} != {(n, self.Hq, self.d)}")
        out = torch.empty((n, self.Hq, self.d), dtype=torch.float32, device=q.device) \
            if out is None else out
        self._check(_lib.kvq_decode_naive(self._ctx, layer, n, _i32(seq_ids),
                                          _dev(q, torch.float16, "q"),
                                          _out(out, (n, self.Hq, self.d), torch.float32, q.device,
                                               "out"), _stream()),
                    "kvq_decode_naive")
        return out

    def dense_decode(self, seq_lens, q, k, v, out=None):
        """Dense FP16 attention over a device-resident cache (comparator).
        q fp16 [n, Hq, d]; k, v fp16 [n, max_tokens, Hkv, d]; returns out f32."""
        import torch
        n = len(seq_lens)
        if q.shape != (n, self.Hq, self.d):
            raise ValueError(f"q shape {tuple(q.shape)} != {(n, self.Hq, self.d)}")
        want = (n, self.cfg.max_tokens, self.Hkv, self.d)
        if tuple(k.shape) != want or tuple(v.shape) != want:
            raise ValueError(f"k/v shape must be {want}")
        out = torch.empty((n, self.Hq, self.d), dtype=torch.float32, device=q.device) \
            if out is None else out
        if k.device != q.device or v.device != q.device:
            raise ValueError("q, k and v must be on one device")
        self._check(_lib.kvq_dense_decode(self._ctx, n, _i32(seq_lens),
                                          _dev(q, torch.float16, "q"), _dev(k, torch.float16, "k"),
                                          _dev(v, torch.float16, "v"),
                                          _out(out, (n, self.Hq, self.d), torch.float32, q.device,
                                               "out"), _stream()),
                    "kvq_dense_decode")
        return out

    def export_tier1(self, layer, seq, g):
        """Tier 1 of one (layer, slot, KV head) in plain layouts (numpy)."""
        nbytes = _lib.kvq_tier1_export_bytes(self._ctx, layer, seq)
        if nbytes < 0:
            raise KvqError(int(nbytes), "kvq_tier1_export_bytes")
        buf = np.empty(nbytes, np.uint8)
        self._check(_lib.kvq_export_tier1(self._ctx, layer, seq, g, buf.ctypes.data_as(P), nbytes),
                    "kvq_export_tier1")
        T = self.seq_len(layer, seq)
        NB = (T + 63) // 64
        d = self.d
        out = {}
        o = 0

        def take(name, count, dtype, shape):
            nonlocal o
            nb = count * np.dtype(dtype).itemsize
            out[name] = buf[o:o + nb].view(dtype).reshape(shape).copy()
            o += nb
        take("kcode", T * d, np.uint8, (T, d))
        take("kscale", NB * d, np.uint16, (NB, d))
        take("koff", NB * d, np.uint16, (NB, d))
        take("eta", NB, np.float32, (NB,))
        take("vcode", T * d, np.uint8, (T, d))
        take("vscale", T * (d // 32), np.uint16, (T, d // 32))
        take("voff", T * (d // 32), np.uint16, (T, d // 32))
        take("vmin", d, np.float32, (d,))
        take("vmax", d, np.float32, (d,))
        assert o == nbytes
        out["T"], out["d"] = T, d
        return out

    def export_trace(self, which, seq):
        """One per-step array of the last decode step for slot `seq` (numpy)."""
        code = TR[which]
        nbytes = _lib.kvq_trace_bytes(self._ctx, code, seq)
        if nbytes < 0:
            raise KvqError(int(nbytes), "kvq_trace_bytes")
        arr = np.empty(nbytes // np.dtype(_TR_DTYPE[which]).itemsize, _TR_DTYPE[which])
        self._check(_lib.kvq_export_trace(self._ctx, code, seq, arr.ctypes.data_as(P), nbytes),
                    "kvq_export_trace")
        return arr
