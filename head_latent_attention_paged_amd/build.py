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

# Sources and their device-code flags.  Kernels whose loop-carried MFMA accumulators are read
# by VALU code do better with the accumulators in VGPRs (-amdgpu-mfma-vgpr-form); the row-split
# kernel keeps them in AGPRs, which only MFMAs touch inside its loop.
VGPR_FORM = ["-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form"]
SOURCES = {
    "mla_kernels.hip": VGPR_FORM,
    "mla_decode_big.hip": VGPR_FORM,
    "mla_decode_rows.hip": [],
    "mla_decode_fp8.hip": VGPR_FORM,
    "mla_decode_wide.hip": [],
    "mla_api.cpp": [],
    "mla_noalloc.hip": [],
}
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def compile_cmds(objdir: str):
    cmds = []
    for src, extra in SOURCES.items():
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmds.append(([HIPCC, *COMMON, *extra, "-Rpass-analysis=kernel-resource-usage",
                      "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
                      os.path.join(CSRC, src), "-o", obj], obj))
    return cmds


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
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cmds = compile_cmds(objdir)
    procs = [(subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True), c) for c, _ in cmds]
    remarks = []
    failed = False
    for p, c in procs:
        out, err = p.communicate()
        remarks.append(err)
        if p.returncode != 0:
            sys.stderr.write(out + err)
            failed = True
    if failed:
        raise RuntimeError("hipcc failed compiling libmla.so sources")
    tmp = LIB + ".tmp"
    link = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, o in cmds], "-o", tmp],
                          capture_output=True, text=True)
    if link.returncode != 0:
        sys.stderr.write(link.stdout + link.stderr)
        raise RuntimeError("hipcc failed linking libmla.so")
    usage = parse_resource_usage("\n".join(remarks))
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
