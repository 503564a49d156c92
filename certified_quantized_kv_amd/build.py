"""Builds libkvq.so (HIP, gfx950) in-tree with hipcc.

Flags that matter for reproducible decisions:
  -ffp-contract=off                 no implicit fma contraction (hipcc defaults to fast)
  -fno-gpu-flush-denormals-to-zero  fp32 denormals kept
  (IEEE fp32 division stays on: no -ffast-math, no approximate divide)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                    no packed fp32 instructions are generated
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
OBJ = os.path.join(HERE, "_build")

SOURCES = ["kvq_codec.hip", "kvq_score.hip", "kvq_select.hip", "kvq_control.hip",
           "kvq_decode.hip", "kvq_dense.hip", "kvq_api.hip", "kvq_noalloc.hip"]

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-fno-gpu-flush-denormals-to-zero", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def hipcc():
    for p in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.exists(p) or p == "hipcc":
            return p


def build(verbose=False):
    """Compiles every source (always) and links libkvq.so."""
    os.makedirs(OBJ, exist_ok=True)

    def one(src):
        obj = os.path.join(OBJ, src.replace(".hip", ".o"))
        cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            noise = "is not a recognized feature for this target"
            msg = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
            if msg.strip():
                print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
