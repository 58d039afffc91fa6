"""Builds libttt_la.so for gfx950 in-tree with hipcc.

    python -m ttt_weight_layers_amd.build [-v]

Each ``csrc/*.hip`` file is compiled to an object under ``_build/`` and the
objects are linked into ``ttt_weight_layers_amd/libttt_la.so``.  Always
rebuilds (the call is the "does it build" check).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libttt_la.so")
ARCH = "gfx950"

# -packed-fp32-ops keeps hipcc from emitting packed fp32 VALU instructions.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libttt_la.so)")


# Per-file options.  The 32x32-tile kernels (and the delta-rule walk) keep their fp32 state in MFMA
# accumulators that the vector ALUs also scale and convert every chunk; asking
# for the VGPR form of the MFMA results keeps the state in ordinary VGPRs
# instead of AGPRs, which would need a copy for every such operation.
FILE_FLAGS = {
    "chunk_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "swiglu.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "delta.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the gfx feature flag; drop that one harmless warning
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int = 4, out: str = LIB, build_dir: str = BUILD,
          host_flags=(), link_flags=("-Wl,--no-undefined",)) -> str:
    """Compiles every csrc/*.hip into build_dir and links ``out``.  host_flags
    are added to every compile (for options of the host pass only, each must be
    preceded by -Xarch_host); link_flags to the link."""
    cc = hipcc()
    os.makedirs(build_dir, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not sources:
        raise RuntimeError("no HIP sources found")
    objs = []
    cmds = []
    for src in sources:
        obj = os.path.join(build_dir, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmds.append([cc, *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *host_flags, "-c", src,
                     "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = out + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_flags, "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
