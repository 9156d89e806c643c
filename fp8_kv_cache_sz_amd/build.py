"""Build the gfx950 HIP library (libsplitzip.so) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", name) for name in
           ("encode.hip", "decode.hip", "calibrate.hip", "runtime.hip", "transfer.hip")]
HEADERS = [os.path.join(ROOT, "include", "splitzip.h"), os.path.join(HERE, "csrc", "common.hpp")]
LIBRARY = os.path.join(HERE, "libsplitzip.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed-FP32 instructions anywhere (the codec has no float math; this
    # keeps the compiler from ever emitting them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libsplitzip.so (always recompiles)."""
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def is_stale() -> bool:
    if not os.path.exists(LIBRARY):
        return True
    t = os.path.getmtime(LIBRARY)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
