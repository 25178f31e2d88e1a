"""Host-sanitizer build of the C ABI's host code (argument validation, device check).

Builds vc_api.hip with AddressSanitizer and UndefinedBehaviorSanitizer on the host pass only
(the kernels are not instrumented) and links it with the regular kernel objects into a separate
library; the CPU test-suite then runs the ABI's validation paths through it with the clang ASan
runtime preloaded (VC_LIB_PATH selects the library). Not used by the product path."""
from __future__ import annotations

import glob
import os
import subprocess

from . import build as _b

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that matches hipcc's host compiler."""
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not cands:
        raise FileNotFoundError("clang ASan runtime not found under /opt/rocm/llvm")
    return cands[-1]


def build_sanitized(out_dir: str) -> str:
    objdir = os.path.join(_b.HERE, "_build")
    objs = []
    for src in _b.SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        if src == "vc_api.hip":
            obj = os.path.join(out_dir, "vc_api_san.o")
            _b._run([_b.HIPCC] + _b.FLAGS + SAN + ["-c", os.path.join(_b.CSRC, src), "-o", obj], False)
        elif not os.path.exists(obj):
            _b._run([_b.HIPCC] + _b.FLAGS + _b.EXTRA.get(src, []) + ["-c", os.path.join(_b.CSRC, src), "-o", obj], False)
        objs.append(obj)
    lib = os.path.join(out_dir, "libvc_san.so")
    _b._run([_b.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + SAN + objs + ["-o", lib], False)
    return lib


if __name__ == "__main__":
    import sys
    print(build_sanitized(sys.argv[1] if len(sys.argv) > 1 else os.path.join(_b.HERE, "_build")))
