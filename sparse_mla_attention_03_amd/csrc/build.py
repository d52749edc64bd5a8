"""Build libsparsemla.so for gfx950 with hipcc (in-tree, next to this file).

    python -m sparse_mla_attention_03_amd.csrc.build      # or build.build()

The translation units compile in parallel, then link into one shared
library exporting the C ABI of include/sparse_mla.h.  The device-ceiling
probes the benchmark reports beside it (include/smla_ceiling.h) go into a
library of their own, libsmla_ceiling.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsparsemla.so")
SOURCES = ["smla_api.hip", "smla_kernels.hip", "smla_prefill.hip", "smla_rope_cache.hip"]
CEILING_LIB = os.path.join(HERE, "libsmla_ceiling.so")
CEILING_SOURCES = ["smla_ceiling.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: with AGPR accumulators the register allocator
    # shuffles them between AGPR tuples every loop trip; in VGPR form the
    # accumulators stay in place and the row prefetch buffers go to AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", HERE,
]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    objs = []

    def compile_one(src: str) -> str:
        obj = os.path.join(HERE, "_build", src.replace(".hip", ".o"))
        os.makedirs(os.path.dirname(obj), exist_ok=True)
        cmd = [hipcc, *HIPCC_FLAGS, "-c", os.path.join(HERE, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                         if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES) + len(CEILING_SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES + CEILING_SOURCES))
    for lib, o in ((LIB, objs[:len(SOURCES)]), (CEILING_LIB, objs[len(SOURCES):])):
        tmp = lib + ".tmp"
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *o]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link of {os.path.basename(lib)} failed:\n{r.stdout}{r.stderr}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
