"""Build libw4a4.so in-tree with hipcc for gfx950.

    python -m w4a4_post_quantized_amd.build          # or build() from Python

Every source in csrc/ is compiled to an object in _build/ (in parallel) and
linked into w4a4_post_quantized_amd/libw4a4.so.  Always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libw4a4.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", INCLUDE, "-I", CSRC,
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]

SOURCES = ["api.cpp", "transform_quant.hip", "gemm.hip", "gemm_decode.hip", "weights.hip",
           "linear_decode.hip", "kv_cache.hip", "attention.hip", "ternary.hip", "gemm_f6.hip",
           "measure.hip"]


# per-source flags.  gemm.hip: MFMA results in ordinary VGPRs, so the
# one-tile-group fold reads its int32 sums without accumulator-register moves
# (64 v_accvgpr_read per K tile and wave in the 128x128 tile)
SOURCE_FLAGS = {
    "gemm.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, extra=()):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), *extra]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx950 feature flag: drop that warning
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err


def build(verbose: bool = True, extra_flags=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda s: _compile(s, extra_flags), SOURCES))
    objs = []
    for obj, err in results:
        objs.append(obj)
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
