"""Build libmoe.so (the HIP library behind include/moe.h) for gfx950, in-tree.

Every call recompiles: one hipcc per source in parallel, then a shared link.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["api.hip", "route.hip", "align.hip", "tile_gemm.hip", "stream_gemm.hip", "pack.hip",
           "small_layer.hip",
           "quant.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-fvisibility=hidden",
    "-I" + os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l)   # host-pass notice, harmless
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]

    def compile_one(i):
        return _run([HIPCC] + FLAGS + ["-c", os.path.join(CSRC, SOURCES[i]), "-o", objs[i]])

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        logs = list(ex.map(compile_one, range(len(SOURCES))))
    tmp = LIB + ".tmp"
    logs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs))
    os.replace(tmp, LIB)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
