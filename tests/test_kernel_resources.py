"""Compile-time checks of the gfx950 kernels (CPU only; needs hipcc).

A kernel that spills registers to scratch memory still gives correct
results, so the parity tests cannot see it, but a spill inside a main loop
costs a large share of its speed.  These checks compile each kernel source
for gfx950 with the compiler's resource report and require:
  * no scratch memory and no spilled vector registers in any kernel (scalar
    registers spilled into vector-register lanes, without scratch, are
    allowed: the routing kernels for very many experts have a few);
  * the LDS sizes the kernels' pipelines are designed around.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from mixture_experts_layer_38_amd import build

HIPCC = build.HIPCC
pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")),
                                reason="hipcc not available")


def _report(src: str, tmp_path) -> dict[str, dict[str, int]]:
    """Kernel name -> resource fields, from -Rpass-analysis=kernel-resource-usage."""
    cmd = [HIPCC, *build.HIP_FLAGS, "--offload-device-only", "-c", src, "-o", str(tmp_path / "k.o"),
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    out: dict[str, dict[str, int]] = {}
    cur = None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[bytes/(?:lane|block)\])?: (\d+)", line)
        if m and cur is not None:
            out[cur][m.group(1).strip()] = int(m.group(2))
    return out


KERNEL_SOURCES = sorted(f for f in os.listdir(os.path.join(build.CSRC, "kernels")) if f.endswith(".hip"))


@pytest.mark.parametrize("name", KERNEL_SOURCES)
def test_no_scratch_or_spills(name, tmp_path):
    rep = _report(os.path.join(build.CSRC, "kernels", name), tmp_path)
    kernels = {k: v for k, v in rep.items() if "ScratchSize" in v}
    assert kernels, f"no kernel report for {name}"
    bad = {k: (v.get("ScratchSize"), v.get("VGPRs Spill"))
           for k, v in kernels.items()
           if v.get("ScratchSize", 0) or v.get("VGPRs Spill", 0)}
    assert not bad, f"kernels with scratch or spills in {name}: {bad}"


def test_prefill_lds_rings(tmp_path):
    """256-row tiles use all 160 KB of LDS (five 32 KB units); 128-row tiles three 48 KB slots."""
    rep = _report(os.path.join(build.CSRC, "kernels", "ffn_prefill.hip"), tmp_path)
    sizes = {k: v.get("LDS Size") for k, v in rep.items() if "ffn_prefill_kernel" in k}
    assert sizes
    for k, lds in sizes.items():
        if "Li256ELi5E" in k:
            assert lds == 5 * 32768, (k, lds)
        elif "Li128ELi3E" in k:
            assert lds == 3 * 49152, (k, lds)
