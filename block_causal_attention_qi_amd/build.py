"""Build libqi.so (HIP kernels for gfx950 + the host tables) in-tree.

    python -m block_causal_attention_qi_amd.build

Kernels and the C ABI are compiled with hipcc for gfx950 only; the host tables
are compiled with g++ and -ffp-contract=off (each fp32 operation rounded on its
own).  The library lands in block_causal_attention_qi_amd/lib/libqi.so.

The calibration microbenchmarks (include/qi_calib.h) are a separate,
bench-only library, lib/libqi_calib.so: they allocate, create a stream and
block, which the product library never does."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(OUT_DIR, "libqi.so")
CALIB_LIB = os.path.join(OUT_DIR, "libqi_calib.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 ops stay off: hipcc would otherwise form v_pk_* fp32 math
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wno-unused-result",
]
# The attention kernel's translation unit keeps MFMA accumulators in VGPRs
# (two waves per SIMD share the VGPR file with the softmax state).
ATTN_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    if os.path.exists(LIB):
        os.remove(LIB)  # a failed build must not leave an older library behind
    obj_dir = os.path.join(OUT_DIR, "obj")
    os.makedirs(obj_dir, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    host_obj = os.path.join(obj_dir, "host_tables.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-c",
          os.path.join(CSRC, "host_tables.cpp"), "-o", host_obj])
    objs.append(host_obj)
    api_obj = os.path.join(obj_dir, "qi_api.o")
    out = _run([hipcc, *HIP_FLAGS, "-c", os.path.join(CSRC, "qi_api.hip"), "-o", api_obj])
    attn_obj = os.path.join(obj_dir, "attention.o")
    out += _run([hipcc, *HIP_FLAGS, *ATTN_FLAGS, "-c", os.path.join(CSRC, "attention.hip"), "-o", attn_obj])
    if verbose and out.strip():
        print(out)
    objs.append(api_obj)
    objs.append(attn_obj)
    na_obj = os.path.join(obj_dir, "noalloc.o")
    _run([hipcc, *HIP_FLAGS, "-c", os.path.join(CSRC, "noalloc.hip"), "-o", na_obj])
    objs.append(na_obj)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    build_calib(hipcc, obj_dir)
    return LIB


def build_calib(hipcc: str, obj_dir: str) -> str:
    """The bench-only calibration library (its own .so, not linked into
    libqi.so)."""
    if os.path.exists(CALIB_LIB):
        os.remove(CALIB_LIB)
    calib_obj = os.path.join(obj_dir, "calib.o")
    _run([hipcc, *HIP_FLAGS, "-c", os.path.join(CSRC, "calib.hip"), "-o", calib_obj])
    tmp = CALIB_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", calib_obj, "-o", tmp])
    os.replace(tmp, CALIB_LIB)
    return CALIB_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
