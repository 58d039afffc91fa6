"""Builds a host-sanitized copy of libttt_la.so for the host-only tests.

    python -m ttt_weight_layers_amd.build_sanitized [-v]

The host code of every csrc/*.hip file is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer (device code is built as usual and is never run by
those tests); the objects go to _build/sanitized/ and the library to
_build/sanitized/libttt_la_san.so.  It is loaded by setting TTT_LA_LIBRARY to
that path and preloading the sanitizer runtime (``runtime()``) into the
process, which is not itself built with the sanitizer.
"""
from __future__ import annotations

import glob
import os
import sys

from . import build as _b

OUT_DIR = os.path.join(_b.BUILD, "sanitized")
LIB = os.path.join(OUT_DIR, "libttt_la_san.so")

HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
              "-Xarch_host", "-g"]
# the sanitizer runtime comes from the preloaded library, not from the link
LINK_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"]


def runtime() -> str:
    """Path of the clang AddressSanitizer runtime (it also carries the UBSan handlers)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")) + \
        sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/x86_64-unknown-linux-gnu/libclang_rt.asan.so"))
    if not hits:
        raise RuntimeError("clang AddressSanitizer runtime not found under /opt/rocm/llvm")
    return hits[-1]


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    srcs = glob.glob(os.path.join(_b.CSRC, "*")) + glob.glob(os.path.join(_b.INCLUDE, "*.h"))
    return any(os.path.getmtime(f) > t for f in srcs)


def build(verbose: bool = False, jobs: int = 8) -> str:
    return _b.build(verbose=verbose, jobs=jobs, out=LIB, build_dir=OUT_DIR, host_flags=HOST_FLAGS,
                    link_flags=LINK_FLAGS)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
