"""Host-sanitizer build of libvda for the CPU tests of the C ABI.

    python -m frame_wise_delta_amd.build_sanitized

Compiles the host code of the ABI (``csrc/vda_api.hip``: validation, index
maps, workspace sizing, launch set-up) with AddressSanitizer and
UndefinedBehaviorSanitizer on the host side only (the device code of that
file is built as usual), links it with the regular objects of the other
sources (which ``build.py`` leaves in ``_build/``) and writes
``_build/san/libvda_san.so``.  A process that loads it needs the clang ASan
runtime preloaded; ``runtime()`` returns its path.
"""
from __future__ import annotations

import os
import subprocess

from . import build as b

SAN_DIR = os.path.join(b.BUILD, "san")
LIB = os.path.join(SAN_DIR, "libvda_san.so")
CLANG = "/opt/rocm/llvm/bin/clang++"


def runtime() -> str:
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.exists(path):
        raise RuntimeError("clang ASan runtime not found")
    return path


def build_sanitized() -> str:
    os.makedirs(SAN_DIR, exist_ok=True)
    api = os.path.join(b.CSRC, "vda_api.hip")
    others = [os.path.join(b.BUILD, n) for n in ("vda_attn.o", "vda_prepare.o", "vda_readout.o", "vda_scan.o")]
    if not all(os.path.exists(o) for o in others):
        b.build()
    obj = os.path.join(SAN_DIR, "vda_api_san.o")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
    b._run([b.hipcc(), *b.CFLAGS, *host_san, "-c", api, "-o", obj])
    tmp = LIB + ".tmp"
    b._run([CLANG, "-shared", "-fsanitize=address,undefined", "-shared-libsan", "-o", tmp, obj, *others,
            "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_sanitized())
