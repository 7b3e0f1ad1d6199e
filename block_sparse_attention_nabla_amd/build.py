"""Build libnabla.so (gfx950) in-tree with hipcc.

Usage: python -m block_sparse_attention_nabla_amd.build
Each translation unit is compiled to an object under ``_build/`` in parallel,
then linked into ``block_sparse_attention_nabla_amd/libnabla.so``.
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
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnabla.so")
ARCH = "gfx950"

SOURCES = [
    "validate.cpp",
    "nabla_api.cpp",
    "mask_kernels.hip",
    "schedule.hip",
    "attn_fwd.hip",
    "attn_bwd.hip",
    "reorder.hip",
    "fidelity.hip",
    "static_scratch.hip",
]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-function",
    # Keep the compiler from forming packed-fp32 VALU ops (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + HIPCC_FLAGS + lang + ["-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature.
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stderr or "").splitlines() if noise not in ln and ln.strip()]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
