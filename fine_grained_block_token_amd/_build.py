"""Build libfgfp8.so (the HIP library) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfgfp8.so")
SOURCES = ["abi.hip", "cast.hip", "gemm.hip", "gemm_wide.hip"]
OBJDIR = os.path.join(PKG, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# MFMA results in VGPRs (the promotion reads them with VALU instructions); the wide
# kernel keeps its 256 accumulators per lane in the accumulation registers instead
VGPR_FORM = ["-mllvm", "--amdgpu-mfma-vgpr-form"]
NO_VGPR_FORM = {"gemm_wide.hip"}


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def flags_for(src: str):
    return HIPCC_FLAGS + ([] if os.path.basename(src) in NO_VGPR_FORM else VGPR_FORM)


def build(verbose: bool = False) -> str:
    """Compile each source to an object with its own flags (in parallel), then link."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJDIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    jobs = []
    for src in sources():
        obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
        cmd = [hipcc, *flags_for(src), *inc, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    errors = []
    for obj, proc in jobs:
        out, err = proc.communicate()
        if proc.returncode != 0:
            errors.append(out + err)
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
