"""Ahead-of-time build of the HIP library for gfx950.

`python -m moe_grouped_gemm_fp8_amd.build` compiles every source under csrc/
into moe_grouped_gemm_fp8_amd/libfg8.so with hipcc.  Packed FP32 VALU
instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfg8.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the promotion FMAs read them directly instead of
    # copying each one out of AGPRs first.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # Kernel arguments that fit in 16 SGPRs are preloaded by the hardware at
    # wave launch instead of loaded by the kernel's first instructions.
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def compile_shared(srcs, out, extra=()):
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, *srcs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}) building {out}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, out)
    return out


def build_library():
    return compile_shared(sources(), LIB)


def build_probes():
    d = os.path.join(ROOT, "tests", "gpu_probes")
    return compile_shared([os.path.join(d, "probes.hip")], os.path.join(d, "libfg8_probes.so"))


if __name__ == "__main__":
    print(build_library())
    print(build_probes())
