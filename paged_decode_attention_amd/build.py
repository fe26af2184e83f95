"""Build libkvq.so (the HIP kernels and C-ABI entry points) in-tree for gfx950.

``python -m paged_decode_attention_amd.build`` compiles every source under
``csrc/`` with hipcc and links ``paged_decode_attention_amd/libkvq.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkvq.so")

SOURCES = ["kvq_api.cpp", "kvq_store.hip", "kvq_decode.hip", "kvq_gqa_mfma.hip", "kvq_merge.hip", "kvq_mla.hip",
           "kvq_noalloc.hip"]

ARCH = "gfx950"
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-I" + os.path.join(ROOT, "include"),
    # never let the compiler form packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source additions.  The separate-K/V matrix-core kernel keeps its MFMA
# accumulators in ordinary VGPRs: it then needs no AGPR copies and fits two
# (head_dim 256) or three (head_dim 128) waves per SIMD.  The MLA kernel, whose
# output accumulator fills the AGPR file, keeps the default.
EXTRA_FLAGS = {
    "kvq_gqa_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkvq.so)")


# Compilation units: (source, object name, defines).  The VALU decode kernels
# are compiled once per storage type (0 bf16, 1 e4m3, 2 q8_0, 3 e4m3 cast,
# 4 e5m2 cast), so that their objects build in parallel.
UNITS = [(src, os.path.splitext(src)[0], []) for src in SOURCES if src != "kvq_decode.hip"] + [
    ("kvq_decode.hip", "kvq_decode_qt%d" % qt, ["-DKVQ_DECODE_QT=%d" % qt]) for qt in range(5)]


def _compile(unit) -> str:
    src, name, defines = unit
    obj = os.path.join(BUILD_DIR, name + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA_FLAGS.get(src, []), *defines, "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(UNITS), max(1, (os.cpu_count() or 1)))
    # the longest units first
    order = sorted(UNITS, key=lambda u: u[0] not in ("kvq_decode.hip", "kvq_gqa_mfma.hip",
                                                     "kvq_mla.hip"))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, order))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
