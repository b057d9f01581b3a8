"""Build libpic.so in-tree with hipcc for gfx950.

Usage: python -m position_independent_kv_amd.build   (or call build()).
Also builds the host-only part with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer (``libpic_host_san.so``'s companion test binary is
built by the tests themselves).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpic.so")

SOURCES = ["pic_attn.hip", "pic_table.hip", "pic_cache.hip", "pic_stream.hip", "pic_host.cpp",
           "pic_spans.cpp", "pic_sched.cpp"]
HEADERS = ["pic_common.hpp", "pic_device.hpp", "pic_host.hpp"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # packed fp32 VALU instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for c in [os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")]:
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libpic.so)")


def build(verbose: bool = False) -> str:
    """Compile every source into libpic.so (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
