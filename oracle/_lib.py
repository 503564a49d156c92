"""ctypes loader for the C half of the oracle (``oracle/oracle.c``).

Test infrastructure only: loaded by tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The HIP product library never loads it.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11"]


def build(force=False):
    """Compile liboracle.so with gcc (fp contraction off, no fast-math)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None

P = ctypes.c_void_p
I = ctypes.c_int
I64 = ctypes.c_int64
F = ctypes.c_float

_SIGS = {
    "orc_h2f": (F, [ctypes.c_uint16]),
    "orc_f2h": (ctypes.c_uint16, [F]),
    "orc_ru16": (ctypes.c_uint16, [F]),
    "orc_exp2k": (F, [F]),
    "orc_exp2k_coeffs": (None, [P]),
    "orc_exp2k_vec": (None, [I64, P, P]),
    "orc_quant_key_block": (None, [I, I, P, P, P, P]),
    "orc_quant_value_token": (F, [I, P, P, P, P]),
    "orc_build_tier1": (None, [I, I, P, P, P, P, P, P, P, P, P, P, P]),
    "orc_query_scale": (F, [I]),
    "orc_query": (None, [I, I, P, P]),
    "orc_int8_block": (None, [I, I, I, P, P, P, P, P, I64, P]),
    "orc_fp16_scores": (None, [I, I, I, P, P, P]),
    "orc_int8_scores": (None, [I, I, I, P, P, P, P, P, P]),
    "orc_ingredients": (None, [I, P, P, P]),
    "orc_weights": (None, [I, P, P, P, P]),
    "orc_gfactors": (None, [I, P, P, P]),
    "orc_attend": (None, [I, I, I, P, P, P]),
    "orc_value_rows": (None, [I, I, P, P, P, P, P, P]),
}


def lib():
    global _lib
    if _lib is None:
        # a sanitizer build of the same source (tests/test_oracle_asan.py)
        path = os.environ.get("KVQ_ORACLE_LIB") or build()
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def ptr(a):
    """Raw data pointer of a C-contiguous numpy array (None for None)."""
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def c_array(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)
