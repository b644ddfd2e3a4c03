"""Build libfp8bw.so in-tree for gfx950 with hipcc.

    python -m blockwise_scaled_fp8_amd.build

Compiles every source under csrc/ into _build/ (at the repository root) and
links blockwise_scaled_fp8_amd/libfp8bw.so.  Flags: gfx950 only, -O3, no
fast-math (IEEE fp32 division stays correctly rounded, which the quantizer's
scale and reciprocal depend on), hidden visibility except the C ABI, and
packed-fp32 instruction selection disabled.
"""

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfp8bw.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["quant.hip", "gemm.hip", "api.cpp"]
# Per-source extra flags.  gemm.hip: select the VGPR form of MFMA so the
# rescale's VALU reads the MFMA results without AGPR->VGPR copies.
EXTRA = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops" not in line and "is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return out


def build(verbose=False, jobs=None):
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC, *FLAGS, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src),
                     "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs or min(8, len(cmds))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    out = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
