"""Build libmk.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

The kernels are compiled as six translation units of kernels.hip (one per batch size, plus probes and
dispatch) in parallel, with api.cpp and graph.cpp, then linked into one shared library.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmk.so")
SOURCES = ["kernels.hip", "api.cpp", "graph.cpp"]
HEADERS = ["mk_internal.h", "graph.h", "gemv_stream.inc", "schedule_table.inc"]
BATCHES = [1, 2, 4, 8, 16]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
FLAGS = ["-O3", "--offload-arch=gfx950", "-fPIC", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]


def _units(tmp):
    inc = ["-I", os.path.join(HERE, "..", "include")]
    k = os.path.join(CSRC, "kernels.hip")
    units = [(["-c", k], os.path.join(tmp, "kernels_common.o"))]
    units += [([f"-DMK_NB={nb}", "-c", k], os.path.join(tmp, f"kernels_b{nb}.o")) for nb in BATCHES]
    units += [(["-c", os.path.join(CSRC, f)], os.path.join(tmp, f + ".o")) for f in ("api.cpp", "graph.cpp")]
    return [(["hipcc", *FLAGS, *inc, *args, "-o", out], out) for args, out in units]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line)
    return r.returncode, " ".join(cmd), err


def build(verbose: bool = False, extra=(), jobs: int = 0, out: str = LIB) -> str:
    """Compile and link the library to `out` (default: the in-tree libmk.so).  extra: additional
    hipcc arguments, e.g. -D options that select a measured alternative (see VARIANTS)."""
    tmp = tempfile.mkdtemp(prefix="mkbuild_")
    try:
        units = _units(tmp)
        units = [(cmd[:1] + list(extra) + cmd[1:], obj) for cmd, obj in units]
        jobs = jobs or min(len(units), max(1, min(os.cpu_count() or 1, 16)))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, [c for c, _ in units]))
        for rc, cmd, err in results:
            if verbose:
                print(cmd, flush=True)
            if rc != 0:
                raise RuntimeError(f"hipcc failed ({rc}): {cmd}\n{err}")
            if verbose and err.strip():
                print(err)
        link = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, o in units], "-o", out + ".tmp"]
        rc, cmd, err = _run(link)
        if verbose:
            print(cmd, flush=True)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}): {cmd}\n{err}")
        os.replace(out + ".tmp", out)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return out


# Compile-time alternatives that the offline measurements compare with the built default:
# the GEMV pipeline depth and group size (DEPTH groups of CG 16-byte chunks per lane in flight per
# wave) and the counter form of events.
VARIANTS = {
    "depth1": ["-DMK_GEMV_DEPTH=1"],
    "depth3": ["-DMK_GEMV_DEPTH=3"],
    "counter_events": ["-DMK_EVENT_COUNTER=1"],
    "cg2": ["-DMK_GEMV_CG=2"],
    "cg2d4": ["-DMK_GEMV_CG=2", "-DMK_GEMV_DEPTH=4"],
}
VARIANT_DIR = os.path.join(HERE, "variants")


def build_variant(name: str, verbose: bool = False) -> str:
    """Build variants/libmk_<name>.so; load it by setting MK_LIBRARY to its path."""
    os.makedirs(VARIANT_DIR, exist_ok=True)
    return build(verbose, VARIANTS[name], out=os.path.join(VARIANT_DIR, f"libmk_{name}.so"))


def sources_newer_than_lib() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    inc = os.path.join(HERE, "..", "include", "mk.h")
    return any(os.path.getmtime(os.path.join(CSRC, f)) > t for f in SOURCES + HEADERS) or os.path.getmtime(inc) > t


if __name__ == "__main__":
    if sys.argv[1:2] == ["--variants"]:
        for name in sys.argv[2:] or VARIANTS:
            print(build_variant(name, verbose=True))
    else:
        build(verbose=True, extra=sys.argv[1:])
