"""Build libmoe.so (HIP, gfx950) in-tree.

    python -m bit_dequant_expert_route_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = [os.path.join(CSRC, f) for f in ("moe_kernels.hip", "moe_down.hip", "moe_batch.hip",
                                           "moe_util.hip", "moe_gdn.hip", "moe_api.cpp")]
HEADERS = [os.path.join(CSRC, "moe_internal.h"), os.path.join(CSRC, "moe_device.h"),
           os.path.join(CSRC, "moe_sortnet.h"), os.path.join(CSRC, "moe_launch.h"),
           os.path.join(os.path.dirname(HERE), "include", "moe.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms stay off (the compiler would otherwise form them
    # from scalar float code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(out: str = LIB, extra=()) -> str:
    """Compile every source to an object (in parallel), then link the library."""
    os.makedirs(BUILD, exist_ok=True)
    tag = os.path.splitext(os.path.basename(out))[0]

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD, f"{tag}.{os.path.basename(src)}.o")
        subprocess.run([HIPCC, *FLAGS, *extra, "-c", src, "-o", obj], check=True)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out + ".tmp"],
                   check=True)
    os.replace(out + ".tmp", out)
    return out


def is_stale(lib: str = LIB) -> bool:
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    return any(os.path.getmtime(f) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(), file=sys.stderr)
