"""Build libattn.so (HIP kernels + C-ABI front end) for gfx950 with hipcc.

Run as ``python -m online_softmax_10_amd.build`` or through
``__graft_entry__.build()``.  The library is written next to this file so that
it travels with the source tree.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["attn_api.cpp", "attn_plan.cpp", "attn_bf16.hip", "attn_noalloc.hip", "attn_f32.hip", "attn_decode.hip",
           "online_softmax.hip", "softmax_xent.hip", "attn_kv_outer.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    # Keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Kernel arguments arrive preloaded in SGPRs: a workgroup's first address
    # computations need not wait for a scalar load of the argument block
    # (attention: -0.3 % per launch on 2x16x4096^2 causal, -1 % on 4x8x1024^2).
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", INCLUDE,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        # the host pass does not know the packed-fp32 target feature; everything else is shown
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if lines:
            print(f"[{src}]\n" + "\n".join(lines), file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
