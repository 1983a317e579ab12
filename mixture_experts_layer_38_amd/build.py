"""Build libmoe.so (HIP, gfx950) in-tree.

    python -m mixture_experts_layer_38_amd.build

Every .hip source is compiled with hipcc for gfx950 only, then linked into one
shared library next to this file.  Packed fp32 VALU instructions are disabled
(-packed-fp32-ops): the kernels use plain fp32 arithmetic and MFMA.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libmoe.so")
PEAKS_SRC = os.path.join(CSRC, "peaks", "peaks.hip")
PEAKS_LIB_PATH = os.path.join(HERE, "libmoepeaks.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def sources() -> list[str]:
    out = [os.path.join(CSRC, "moe_api.hip")]
    kdir = os.path.join(CSRC, "kernels")
    out += sorted(os.path.join(kdir, f) for f in os.listdir(kdir) if f.endswith(".hip"))
    return out


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *HIP_FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip())
    if verbose and warn:
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """libmoe.so (the layer) and libmoepeaks.so (the measurement probes)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources() + [PEAKS_SRC]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    peaks_obj = objs.pop()
    for out, inputs in ((LIB_PATH, objs), (PEAKS_LIB_PATH, [peaks_obj])):
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *inputs, "-o", out + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
