"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer build of the C ABI
layer: the host sources (argument validation, workspace carving, dispatch)
are compiled with the sanitizers for the host pass only and linked with the
regular objects of the HIP kernels into _build/asan/libhstu_asan.so.  The
CPU test tier loads it under the clang ASan runtime and runs the ABI tests
(every call there returns before any device work).  Not used on a GPU."""
from __future__ import annotations

import glob
import os
import subprocess

from . import build as hb

ASAN_DIR = os.path.join(hb.BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libhstu_asan.so")
HOST_SOURCES = ("api.cpp", "profile.cpp", "noalloc.hip")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def runtime() -> str:
    """The clang ASan runtime that matches hipcc's compiler (for LD_PRELOAD)."""
    out = subprocess.run(["hipcc", "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        hits = glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        path = hits[0] if hits else ""
    return path


def build() -> str:
    hb.build()  # the regular objects
    os.makedirs(ASAN_DIR, exist_ok=True)
    objs = []
    for src in hb.sources():
        base = os.path.basename(src)
        if base in HOST_SOURCES:
            obj = os.path.join(ASAN_DIR, base + ".o")
            cmd = ["hipcc", "-x", "hip", "-c", src, "-o", obj] + hb.FLAGS + SAN
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError("hipcc (sanitized host pass) failed for %s:\n%s" % (src, r.stderr[-4000:]))
            objs.append(obj)
        else:
            objs.append(os.path.join(hb.BUILD, base + ".o"))
    cmd = ["hipcc", "-shared", "-fPIC", "--offload-arch=" + hb.ARCH, "-o", ASAN_LIB] + objs + \
        ["-shared-libsan", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link (sanitized) failed:\n" + r.stderr[-4000:])
    return ASAN_LIB
