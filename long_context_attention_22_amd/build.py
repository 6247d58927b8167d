"""Build the HIP library (csrc/*.hip, csrc/capi.cpp) for gfx950 into liblca.so.

    python -m long_context_attention_22_amd.build

hipcc cross-compiles without a GPU.  Packed-fp32 instructions are disabled
(-packed-fp32-ops) for every device compile.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblca.so")
OBJ = os.path.join(ROOT, "_build", "lca")

SOURCES = ["kv_compress.hip", "indexer.hip", "topk.hip", "attn.hip", "gemm.hip", "cache.hip", "capi.cpp"]
# MFMA accumulators stay in VGPRs (-amdgpu-mfma-vgpr-form): the kernels keep their accumulators
# within 256 VGPRs, and AGPR accumulators made the compiler copy them back and forth around the
# attention loop's conditional rescale.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-I", os.path.join(ROOT, "include")]
# Per-source additions.  attn.hip: its softmax never sees a NaN, and without the NaN guarantee
# every fmaxf of a value moved across lanes gets an extra canonicalising max.
# indexer.hip: its scores are finite, and without the guarantee every ReLU of an MFMA result costs
# a canonicalising max besides the max with zero.
EXTRA = {"attn.hip": ["-fno-honor-nans"], "indexer.hip": ["-fno-honor-nans"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, src + ".o")
    lang = ["-x", "hip"]
    cmd = ["hipcc", *FLAGS, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    warn = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if warn and verbose:
        print("\n".join(warn), file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
