"""Build libgdn2.so (HIP, gfx950) in-tree.

    python -m gated_delta_rule_07_amd.build

compiles every source under csrc/ with hipcc for gfx950 and links
gated_delta_rule_07_amd/libgdn2.so.  Packed-FP32 instruction selection is
switched off for device code (the flag is harmless for the host pass).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libgdn2.so")
BUILD = os.path.join(HERE, "_build")
ARCH = os.environ.get("GDN2_OFFLOAD_ARCH", "gfx950")

SOURCES = ["gdn2_api.cpp", "gdn2_recurrent.hip", "gdn2_chunk.hip", "gdn2_fused.hip", "gdn2_bwd.hip", "gdn2_segment.hip",
           "gdn2_rule_r1.hip"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument"]
# Per-file flags.  The segment map's state loop carries its matrix-core
# accumulators from chunk to chunk and scales them on the vector ALU; by
# default the compiler keeps them in AGPRs and copies them to VGPRs and back
# every chunk, which the VGPR form of the products avoids.
EXTRA = {"gdn2_segment.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [_hipcc(), *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    r = subprocess.run([_hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
