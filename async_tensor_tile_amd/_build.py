"""Build the gfx950 shared library in-tree with hipcc.

Every *.hip file under csrc/ is compiled for gfx950 only and linked into
``libatt_amd.so`` next to this file.  No JIT cache is used, so the built
library travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(HERE, "libatt_amd.so")
# The debug build (ATT_DEBUG): LDS images and ring stages are poisoned before
# they are loaded, the bytes a box's waves issue are checked against the box
# bytes and a barrier's state against its completed phase when its box is
# consumed; failures are recorded for tile_device_status.
OBJ_DEBUG = os.path.join(ROOT, "_build", "obj_debug")
LIB_DEBUG = os.path.join(HERE, "libatt_amd_debug.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    # packed-fp32 instructions stay off (hand-written and compiler-made)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # hardware float atomics for the reduce-add store
    "-munsafe-fp-atomics",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str, debug: bool) -> str:
    obj = os.path.join(OBJ_DEBUG if debug else OBJ, os.path.basename(src) + ".o")
    subprocess.check_call([HIPCC, *FLAGS, *(["-DATT_DEBUG"] if debug else []), "-c", src, "-o", obj])
    return obj


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile every HIP source and link libatt_amd.so (libatt_amd_debug.so
    with debug=True); returns its path."""
    os.makedirs(OBJ_DEBUG if debug else OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    workers = max(1, min(len(srcs), 8))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda f: _compile(f, debug), srcs))
    lib = LIB_DEBUG if debug else LIB
    tmp = lib + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    import sys
    build(verbose=True, debug="--debug" in sys.argv[1:])
