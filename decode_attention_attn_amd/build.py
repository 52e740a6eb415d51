"""Build libmfa.so (gfx950) in-tree with hipcc.

    python -m decode_attention_attn_amd.build [--isa]

Objects go to _build/ at the repository root; the shared library is written
next to this file, where the Python binding loads it. ``--isa`` also keeps the
AMD assembly of the kernels (``_build/*.s``) for inspection.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmfa.so")
SOURCES = ["attn.hip", "attn_mt.hip", "proj.hip", "probe.hip", "mfa_api.cpp"]
# Per-source extra flags. The attention and GEMM kernels keep their
# accumulators in ordinary VGPRs as MFMA operands: with accumulators in AGPRs
# the compiler copied all of them to VGPRs on every loop iteration, for the
# rarely taken online-softmax rescale in attention (measured: 4-8% of the
# attention kernel's time) and across the two fragment sets of the pipelined
# GEMM loop.
EXTRA = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "proj.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed-fp32 VALU ops are disabled for all device code: the compiler would
# otherwise form v_pk_{add,mul,fma}_f32 from ordinary float code.
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}")
    return out


def build(isa: bool = False, verbose: bool = False) -> str:
    """Compile every source and link libmfa.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD, src + ".o")
        cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + ["-c", path, "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip"]
            if isa:
                cmd += ["-save-temps=obj"]
        out = _run(cmd)
        if verbose and out:
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--isa", action="store_true")
    ap.add_argument("-v", action="store_true")
    args = ap.parse_args()
    print(build(isa=args.isa, verbose=args.v))
