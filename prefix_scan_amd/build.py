"""Build ``prefix_scan_amd/libscan.so`` from the HIP sources in ``csrc/``.

    python -m prefix_scan_amd.build        # or: python prefix_scan_amd/build.py

The library is compiled for gfx950 only, with hipcc, into the package
directory, where the Python binding loads it.  Each source compiles to an
object of its own, several at a time, and the objects are linked into one
shared library.
"""
import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libscan.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # No packed fp32 instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Keep single-lane atomics as written: the wave-aggregating rewrite makes
    # the ticket draw wait for every load issued before it.
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
]


def sources(csrc=CSRC):
    return sorted(glob.glob(os.path.join(csrc, "*.hip")))


def _jobs():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16, int(os.environ.get("MAX_JOBS", n))))


def build(verbose: bool = False, csrc: str = CSRC, out: str = LIB, defines=()) -> str:
    """Compile every *.hip of `csrc` into the shared library `out`; returns
    its path.  `defines` are extra -D options for every source."""
    tmp = out + ".tmp%d" % os.getpid()
    objdir = tempfile.mkdtemp(prefix="libscan_obj")
    extra = ["-D" + d for d in defines]

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [HIPCC] + FLAGS + extra + ["-I", INCLUDE, "-I", csrc, "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    try:
        with ThreadPoolExecutor(_jobs()) as pool:
            objs = list(pool.map(compile_one, sources(csrc)))
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    except BaseException:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
