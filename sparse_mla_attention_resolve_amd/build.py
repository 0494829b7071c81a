"""Build libsmla.so in-tree with hipcc for gfx950.

    python -m sparse_mla_attention_resolve_amd.build [--verbose] [--resource-usage]

Compiles every csrc/*.hip to an object in csrc/_build/ and links them into
sparse_mla_attention_resolve_amd/libsmla.so. Always recompiles, also where a built
library is already present.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(CSRC, "_build")
LIB = os.path.join(HERE, "libsmla.so")
ROOT = os.path.dirname(HERE)

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Wno-unused-variable", "-I", os.path.join(ROOT, "include"),
    # packed fp32 VALU ops stay off: the compiler may not form v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libsmla")


# Per-file code-generation options.
#  -amdgpu-mfma-vgpr-form: the decode kernels hold their MFMA accumulators in VGPRs; left to
#   its heuristics the compiler keeps them in AGPRs and copies them every loop iteration.
#  -fno-honor-nans: the decode kernels never produce or test NaN (masked scores are -inf),
#   so max needs no NaN-quieting instructions around it; infinities keep their semantics.
FILE_FLAGS = {
    "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
}


def _compile(src: str, extra: list[str], verbose: bool) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", ".o"))
    cmd = [hipcc(), *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    return obj, msgs


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, extra, verbose), srcs))
    for _, msgs in results:
        if msgs.strip() and (verbose or resource_usage):
            print(msgs, flush=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    a = ap.parse_args()
    print(build(a.verbose, a.resource_usage))
    sys.exit(0)
