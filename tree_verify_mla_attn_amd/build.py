"""In-tree build of the HIP library ``libkdtree_verify.so`` for gfx950.

Every call recompiles all sources (hipcc cross-compiles without a GPU).  The library
lands next to this file so that it travels with the source tree.

Flags:
  --offload-arch=gfx950                      MI355X only.
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                             no packed-fp32 VALU forms are emitted.
  -mllvm -amdgpu-mfma-vgpr-form=1            MFMAs are selected in their VGPR form, which
                                             lets the register allocator keep the score
                                             accumulator in VGPRs while the 256-register
                                             output accumulator takes the AGPR file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libkdtree_verify.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["attn_bf16.hip", "attn_f32.hip", "prepass.hip", "merge.hip", "ddtree.hip", "sample.hip", "capi.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link ``libkdtree_verify.so``; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
