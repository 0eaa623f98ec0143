"""Build libmoe_gfx950.so in-tree with hipcc for gfx950 (MI355X).

Usage: python -m mixture_experts_expert_moe_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_gfx950.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["route.hip", "route_small.hip", "permute.hip", "gemm.hip", "gemm_big.hip", "combine.hip", "decode.hip",
           "moe_api.cpp"]
# Sources whose kernels issue their own vector loads (inline asm + explicit
# vmcnt waits): their assembly is checked at build time.
ASM_CHECKED = ["gemm_big.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msg))
    if msg.strip():
        print(msg, file=sys.stderr)
    return out


def _check_asm(src: str) -> None:
    from . import asm_check  # build-time only
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".s")
    cmd = [HIPCC, *[f for f in FLAGS if f != "-fPIC"], "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc -S failed for %s:\n%s" % (src, r.stderr[-4000:]))
    problems = asm_check.check_file(out)
    if problems:
        raise RuntimeError("assembly check failed for %s:\n%s" % (src, "\n".join(problems)))


def build() -> str:
    """Compile every HIP/C++ source for gfx950, check the assembly of the
    kernels that manage their own loads, and link the shared library."""
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(ASM_CHECKED))) as ex:
        objs_f = ex.map(_compile, SOURCES)
        checks = [ex.submit(_check_asm, s) for s in ASM_CHECKED]
        objs = list(objs_f)
        for c in checks:
            c.result()
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
