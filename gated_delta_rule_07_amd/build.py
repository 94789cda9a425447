"""Build libgdn2.so (HIP, gfx950) in-tree.

    python -m gated_delta_rule_07_amd.build

compiles every source under csrc/ with hipcc for gfx950 and links
gated_delta_rule_07_amd/libgdn2.so.  Packed-FP32 instruction selection is
switched off for device code (the flag is harmless for the host pass).

It also links libgdn2_hostcheck.so: the same kernels with the host side of
gdn2_api.cpp (argument checks, workspace planning, launch set-up) built with
undefined-behaviour checks that trap (signed overflow, shifts, array bounds,
misaligned or null accesses), for the host-side tests.  The product binding
never loads it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libgdn2.so")
OUT_HOSTCHECK = os.path.join(HERE, "libgdn2_hostcheck.so")
BUILD = os.path.join(HERE, "_build")
ARCH = os.environ.get("GDN2_OFFLOAD_ARCH", "gfx950")

SOURCES = ["gdn2_api.cpp", "gdn2_recurrent.hip", "gdn2_chunk.hip", "gdn2_fused.hip", "gdn2_bwd.hip", "gdn2_segment.hip",
           "gdn2_rule_r1.hip", "gdn2_pad.hip"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument"]
# Per-file flags.  The segment map's state loop carries its matrix-core
# accumulators from chunk to chunk and scales them on the vector ALU; by
# default the compiler keeps them in AGPRs and copies them to VGPRs and back
# every chunk, which the VGPR form of the products avoids.
EXTRA = {"gdn2_segment.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
# Host-only undefined-behaviour traps for the checked build of gdn2_api.cpp
# (each flag after -Xarch_host: device code is compiled as in the product).
HOSTCHECK = [f for x in ("-fsanitize=undefined", "-fsanitize-trap=undefined", "-fsanitize=bounds",
                         "-fno-sanitize-recover=all") for f in ("-Xarch_host", x)]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def _compile(src: str, hostcheck: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ("_hostcheck" if hostcheck else "") + ".o")
    cmd = [_hipcc(), *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [_hipcc(), *COMMON, *(HOSTCHECK if hostcheck else []), "-x", "hip", "-c", os.path.join(CSRC, src),
               "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    r = subprocess.run([_hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        futs = [ex.submit(_compile, src) for src in SOURCES]
        checked_api = ex.submit(_compile, "gdn2_api.cpp", True)
        objs = [f.result() for f in futs]
        api_checked = checked_api.result()
    _link(objs, OUT)
    _link([api_checked if o.endswith("gdn2_api.o") else o for o in objs], OUT_HOSTCHECK)
    if verbose:
        print(f"built {OUT} and {OUT_HOSTCHECK}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
