"""Build libmla.so for gfx950 with hipcc (cross-compiles without a GPU).

The build fails if any kernel uses scratch memory (register spills), unless
MLA_SKIP_SCRATCH_CHECK=1 is set.
"""

from __future__ import annotations

import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmla.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["mla_kernels.hip", "mla_decode_big.hip", "mla_decode_rows.hip", "mla_api.cpp"]


def hipcc_cmd(out: str = LIB):
    return [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form",
            "-Rpass-analysis=kernel-resource-usage",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def parse_resource_usage(text: str):
    """Per-kernel {name: {field: value}} from -Rpass-analysis=kernel-resource-usage remarks."""
    usage, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            usage[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[(?:bytes/lane|waves/SIMD|bytes/block)\])?: (-?\d+)", line)
        if m and cur is not None:
            usage[cur][m.group(1).strip()] = int(m.group(2))
    return usage


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    proc = subprocess.run(hipcc_cmd(tmp), capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError("hipcc failed building libmla.so")
    usage = parse_resource_usage(proc.stderr)
    spills = {k: v for k, v in usage.items() if v.get("ScratchSize", 0) > 0}
    if verbose:
        for k, v in usage.items():
            print(k, {f: v.get(f) for f in ("VGPRs", "AGPRs", "ScratchSize", "Occupancy", "LDS Size")})
    if spills and os.environ.get("MLA_SKIP_SCRATCH_CHECK") != "1":
        os.unlink(tmp)
        raise RuntimeError("kernels use scratch (register spills): %s" % {k: v.get("ScratchSize") for k, v in spills.items()})
    os.replace(tmp, LIB)
    with open(os.path.join(PKG, "resource_usage.txt"), "w") as f:
        for k, v in sorted(usage.items()):
            f.write("%s %s\n" % (k, " ".join("%s=%s" % (a, b) for a, b in sorted(v.items()))))
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print("built", LIB)
