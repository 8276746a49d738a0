"""Build libmk.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmk.so")
SOURCES = ["kernels.hip", "api.cpp", "graph.cpp"]
HEADERS = ["mk_internal.h", "graph.h"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
FLAGS = ["-O3", "--offload-arch=gfx950", "-fPIC", "-shared", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]


def build(verbose: bool = False, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = ["hipcc", *FLAGS, *extra, "-I", os.path.join(HERE, "..", "include"), *srcs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def sources_newer_than_lib() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    inc = os.path.join(HERE, "..", "include", "mk.h")
    return any(os.path.getmtime(os.path.join(CSRC, f)) > t for f in SOURCES + HEADERS) or os.path.getmtime(inc) > t


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
