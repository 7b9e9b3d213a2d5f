"""Build the gfx950 C-ABI library libmoe.so in-tree with hipcc, and the
calibration kernels (libmoe_probe.so, measured instruction rates and HBM read
stream; not part of the layer library).

    python -m sparse_moe_expert_gemv_amd.build        # or build() from Python
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
PROBE_SRC = os.path.join(PKG, "probe", "peak.hip")
PROBE_LIB = os.path.join(PKG, "libmoe_probe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17",
    # never emit packed fp32 VALU ops (v_pk_fma_f32 and friends)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE-correct fp32 division/sqrt (the int8 quantiser divides by amax/127)
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip") or f.endswith(".cpp"))


# host-only C++ (the host expert FFN): g++, vectorised per CPU by function
# multiversioning (target_clones), no HIP
CXX = os.environ.get("CXX", "g++")
CXXFLAGS = ["-O3", "-fPIC", "-std=c++17", "-pthread", "-fno-fast-math", "-mprefer-vector-width=512", "-Wall", "-I", INCLUDE]


# per-file extra flags: MFMA results stay in VGPRs, since the epilogues read every element
# (the int8 FFN after each block, the decode gate/up after each block's seeded sum)
FILE_FLAGS = {"ffn_q8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
              "ffn_float.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    if src.endswith(".cpp"):
        cmd = [CXX, *CXXFLAGS, "-c", src, "-o", obj]
    else:
        cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-pthread", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    build_probe(verbose)
    return LIB


def build_probe(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *CFLAGS, "-mllvm", "-amdgpu-mfma-vgpr-form=1", "-shared", "-o", tmp, PROBE_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (PROBE_SRC, " ".join(cmd), r.stderr))
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print("built", PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
