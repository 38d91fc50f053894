"""Build the gfx950 shared libraries in-tree with hipcc.

libvarq.so          the C-ABI library (include/varq.h): HIP kernels + host API.
libvarq_selftest.so host-only checks of the kernels' scalar arithmetic (CPU tests).

Every HIP translation unit is compiled with IEEE fp32 semantics: no fast math,
no floating-point contraction (fused multiply-adds are written explicitly),
denormals kept, correctly rounded fp32 division, and packed fp32 instructions
disabled.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libvarq.so")
SELFTEST_LIB = os.path.join(HERE, "libvarq_selftest.so")

LIB_SOURCES = ["varq_api.cpp", "quant_pack.hip", "quant_group.hip", "unpack_dequant.hip", "packed_attention.hip"]
SELFTEST_SOURCES = ["quant_math_selftest.cpp"]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src, extra=()):
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIP_FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def _link(objs, out, extra=()):
    tmp = out + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, *extra, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose=False):
    """Compile every HIP source for gfx950 and link libvarq.so and libvarq_selftest.so."""
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        lib_f = [ex.submit(_compile, s) for s in LIB_SOURCES]
        st_f = [ex.submit(_compile, s, ("-mfma",)) for s in SELFTEST_SOURCES]
        lib_objs = [f.result() for f in lib_f]
        st_objs = [f.result() for f in st_f]
    if verbose:
        for _, err in lib_objs + st_objs:
            if err.strip():
                print(err, file=sys.stderr)
    _link([o for o, _ in lib_objs], LIB)
    _link([o for o, _ in st_objs], SELFTEST_LIB, ("-pthread",))
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
