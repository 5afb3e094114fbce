"""Build libra.so (the C-ABI library of gfx950 HIP kernels) in-tree with hipcc.

Usage: ``python -m long_context_exact_tiled_amd.build`` or ``build()`` from Python.
Every source under ``csrc/`` is compiled for gfx950 and linked into
``long_context_exact_tiled_amd/libra.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libra.so")
ROOT = os.path.dirname(PKG)

SOURCES = ["api.hip", "attn_fwd.hip", "attn_fwd_fp8.hip", "attn_bwd.hip", "attn_bwd_f32.hip",
           "fp8_quant.hip", "lse_merge.hip", "ulysses_permute.hip"]

# Packed-fp32 VALU forms are disabled: the compiler may otherwise form them from plain
# float code.  The host pass does not know this device feature and says so (harmless).
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]

# Per-source extras.  The backward's dK/dV kernel runs one wave per SIMD with more than
# 256 registers live; by default the compiler then places the score accumulators in
# AGPRs and copies every element to VGPRs for the softmax VALU work.  The VGPR form of
# the MFMAs keeps them in VGPRs (measured: 910 -> 313 AGPR copies per tile, 4 % faster).
EXTRA = {
    "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def flags_for(src: str) -> list:
    return [*FLAGS, *EXTRA.get(src, [])]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libra)")


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libra.so; returns its path.  Raises on failure."""
    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include")]
    tmp = tempfile.mkdtemp(prefix="libra_build_")
    try:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc, *flags_for(src), *inc, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
            if len(procs) >= jobs:
                _drain(procs, verbose)
        _drain(procs, verbose)
        out_tmp = LIB + ".tmp"
        cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out_tmp, *objs]
        _run(cmd, verbose)
        os.replace(out_tmp, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


def _drain(procs, verbose):
    errors = []
    while procs:
        src, p = procs.pop(0)
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines()
                        if "packed-fp32-ops' is not a recognized feature" not in l)
        if p.returncode != 0:
            errors.append(f"--- {src} ---\n{out}")
        elif verbose and out.strip():
            print(out)
    if errors:
        raise RuntimeError("libra build failed:\n" + "\n".join(errors))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("libra link failed:\n" + r.stdout)


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
