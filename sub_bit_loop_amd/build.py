"""Build libloopvq.so for gfx950 with hipcc (in-tree, no JIT cache).

Every HIP source is compiled with packed-fp32 instructions disabled; the
library links only against the HIP runtime.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libloopvq.so")
# measurement helpers (stream copy / read), kept out of the LoopVQ library
CALIB_LIB = os.path.join(HERE, "libloopvq_calib.so")
CALIB_SOURCES = ["calib.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["encode.hip", "decode.hip", "decode_fast.hip", "decode_half.hip", "decode_gqa.hip", "decode_tasq.hip", "decode_cq.hip",
           "tasq_stats.hip",
           "kmeans.hip", "prefill.hip", "loopvq_api.cpp"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


# The encode kernel orders float keys with v_min/v_med3; with IEEE mode off
# those need no NaN canonicalisation (its inputs are finite by contract).
# The GQA decode kernel keeps its MFMA accumulators in ordinary VGPRs so that
# it fits two waves per SIMD.
EXTRA = {"encode.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee", "-mllvm", "-amdgpu-mfma-vgpr-form"],
         "decode_gqa.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "calib.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src):
    obj = os.path.join(CSRC, "_build", os.path.splitext(src)[0] + ".o")
    os.makedirs(os.path.dirname(obj), exist_ok=True)
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr[-6000:]))
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr[-4000:]))
    os.replace(tmp, lib)


def build(verbose=False):
    srcs = SOURCES + CALIB_SOURCES
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], CALIB_LIB)
    if verbose:
        print("built", LIB, "and", os.path.basename(CALIB_LIB))
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
