"""Build libattn.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: python exact_attention_79_amd/build.py   (or build() from Python; the
package itself refuses to import until the library exists)
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libattn.so")
BUILD_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["attn_api.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip"]

# Packed-fp32 VALU instructions are disabled for all device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-I" + INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


# Measurement programs (not part of the library): source -> executable.
PROBES = {os.path.join(HERE, "probes", "dq_atomic_adds.hip"):
          os.path.join(HERE, "probes", "dq_atomic_adds"),
          os.path.join(HERE, "probes", "valu_rates.hip"):
          os.path.join(HERE, "probes", "valu_rates"),
          os.path.join(HERE, "probes", "dot_precision.hip"):
          os.path.join(HERE, "probes", "dot_precision"),
          os.path.join(HERE, "probes", "mfma_power.hip"):
          os.path.join(HERE, "probes", "mfma_power"),
          os.path.join(HERE, "probes", "halfstep.hip"):
          os.path.join(HERE, "probes", "halfstep")}


def _build_probe(src: str, exe: str):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-munsafe-fp-atomics",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", "-I" + CSRC, src, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
        probes = [ex.submit(_build_probe, s, e) for s, e in PROBES.items()]
        for pr in probes:
            pr.result()
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
