"""CPU runs under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

The oracle's C half and the library's host-side promotion-plan merge are
rebuilt with -fsanitize=address,undefined in a temporary directory and driven
in a child process that preloads the sanitizer runtime: the codec on ragged
lengths and both head dims, scores, block ingredients, weights, the fp64
attention, a whole decode step, and the host merge on random plans.  Any
sanitizer report fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]


def _runtime(cc, name):
    """The sanitizer runtime that matches the compiler of the instrumented code."""
    p = subprocess.run([cc, f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    if p.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"no {name} for {cc}")
    return path


def _child(code, env_extra, tmp_path, runtime):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["PYTHONPATH"] = ROOT + os.pathsep + os.path.join(ROOT, "tests")
    script = tmp_path / "child.py"
    script.write_text(code)
    r = subprocess.run([sys.executable, str(script)], env=env, capture_output=True, text=True,
                       timeout=600)
    report = r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert "CHILD_OK" in r.stdout, r.stdout[-2000:] + report


def test_oracle_under_sanitizers(tmp_path):
    from oracle._lib import CFLAGS, SRC
    lib = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", *CFLAGS, *SAN, SRC, "-o", str(lib), "-lm"])
    code = r'''
import numpy as np
import oracle
from oracle.method import Config
r = np.random.default_rng(3)
for d in (64, 128):
    for T in (1, 63, 64, 65, 200):
        k16 = (r.standard_normal((T, d)) * 3).astype(np.float16).view(np.uint16)
        v16 = r.standard_normal((T, d)).astype(np.float16).view(np.uint16)
        t1 = oracle.build_tier1(k16, v16)
        q16 = r.standard_normal((4, d)).astype(np.float16).view(np.uint16)
        qp = oracle.query(q16)
        shat, delta = oracle.int8_scores(qp, t1)
        sp = oracle.fp16_scores(qp, k16)
        m, L = oracle.ingredients(shat[0])
        W = oracle.weights(m, L)
        gp, gm = oracle.gfactors(delta[0])
        out = oracle.attend(sp, oracle.value_rows(t1, v16))
        res = oracle.decode_step(Config(), q16, [(t1, k16, v16)])
        assert np.all(np.isfinite(res.out))
print("CHILD_OK")
'''
    _child(code, {"KVQ_ORACLE_LIB": str(lib)}, tmp_path, _runtime("gcc", "libasan.so"))


def test_host_merge_under_sanitizers(tmp_path):
    """The host merge of promotion-plan runs (kvq_selftest_merge_runs, no
    device call) from an instrumented build of the library's host code."""
    build = os.path.join(ROOT, "certified_quantized_kv_amd", "build.py")
    import importlib.util
    spec = importlib.util.spec_from_file_location("_kvq_build_san", build)
    kb = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(kb)
    objs = []
    for src in kb.SOURCES:
        obj = tmp_path / src.replace(".hip", ".o")
        flags = list(kb.FLAGS)
        if src == "kvq_api.hip":   # the host logic under test; device code stays as built
            flags += [x for s in SAN for x in ("-Xarch_host", s)]
        subprocess.check_call([kb.hipcc(), *flags, "-c", os.path.join(kb.CSRC, src), "-o", str(obj)],
                              stderr=subprocess.DEVNULL)
        objs.append(str(obj))
    lib = tmp_path / "libkvq.so"
    subprocess.check_call([kb.hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o",
                           str(lib)])
    code = r'''
import ctypes
import numpy as np
lib = ctypes.CDLL(%r)
P = ctypes.c_void_p
lib.kvq_selftest_merge_runs.argtypes = [P, ctypes.c_int64, P, P]
lib.kvq_selftest_merge_runs.restype = ctypes.c_int32
r = np.random.default_rng(5)
for trial in range(300):
    n = int(r.integers(0, 400))
    start = r.integers(0, 4000, n).astype(np.uint64)
    ln = r.integers(1, 50, n).astype(np.uint64)
    grp = r.integers(0, 9, n).astype(np.uint64)
    kind = r.integers(0, 2, n).astype(np.uint64)
    ent = np.ascontiguousarray(ln | (start << 16) | (grp << 32) | (kind << 48), np.uint64)
    out = np.zeros(max(n, 1), np.uint64)
    nout = ctypes.c_int64(-1)
    st = lib.kvq_selftest_merge_runs(ent.ctypes.data_as(P), n, out.ctypes.data_as(P),
                                     ctypes.byref(nout))
    assert st == 0 and 0 <= nout.value <= n, (st, nout.value)
bad = np.array([0], np.uint64)
assert lib.kvq_selftest_merge_runs(bad.ctypes.data_as(P), 1, bad.ctypes.data_as(P),
                                   ctypes.byref(ctypes.c_int64())) != 0
print("CHILD_OK")
''' % str(lib)
    clang = os.path.join(os.path.dirname(os.path.realpath(kb.hipcc())), "..", "lib", "llvm", "bin",
                         "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/lib/llvm/bin/clang"
    _child(code, {}, tmp_path, _runtime(clang, "libclang_rt.asan-x86_64.so"))
