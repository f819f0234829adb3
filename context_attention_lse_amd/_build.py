"""Builds libctxattn.so (hand-written HIP for gfx950) in-tree with hipcc.

Every call recompiles every source. Objects go to ``_build/`` next to this file, the
library to ``libctxattn.so`` in this package directory (written atomically).
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libctxattn.so")
SOURCES = ["api.hip", "attn_bf16.hip", "attn_f32.hip", "merge.hip", "bound.hip", "decode.hip", "copy.hip",
           "segmented.hip", "sinks.hip"]
ARCH = os.environ.get("CTXATTN_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms stay off: the compiler may not emit v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: set HIPCC or install ROCm")


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    return out


# Per-source extra flags. The bf16 step kernel builds without NaN semantics: its inputs are
# finite or -inf (masked scores), and the row maxima then compile to v_max3_f32 with no
# canonicalising moves in front of them.
EXTRA = {"attn_bf16.hip": ["-fno-honor-nans"]}


def build(verbose: bool = False, jobs: int = 6) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        out = _run([cc, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
