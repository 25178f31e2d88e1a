"""Build the HIP shared library ``libvc.so`` for gfx950 in-tree (hipcc, no JIT cache)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libvc.so")
SOURCES = ["vc_api.hip", "vc_quantize.hip", "vc_attention.hip", "vc_cluster.hip", "vc_peak.hip"]
# Per-file extra flags. The attention kernel takes finite inputs by contract: without
# NaN semantics (and with the shader's IEEE mode off) float max needs no operand
# canonicalisation, which removes one VALU op per score element.
# The k-means assignment reads its matrix-core results once each: with the MFMAs in their
# VGPR form it needs no accumulator-register read-back (one vector instruction per distance).
EXTRA = {"vc_attention.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
         "vc_cluster.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",                                   # no implicit FMA: the arithmetic is specified op by op
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(os.path.dirname(HERE), "include"),
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and "--hip-link" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        _run([HIPCC] + FLAGS + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
