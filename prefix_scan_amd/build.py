"""Build ``prefix_scan_amd/libscan.so`` from the HIP sources in ``csrc/``.

    python -m prefix_scan_amd.build        # or: python prefix_scan_amd/build.py

The library is compiled for gfx950 only, with hipcc, into the package
directory, where the Python binding loads it.
"""
import glob
import os
import subprocess
import sys

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
    "-shared",
    "-Wall",
    # No packed fp32 instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Keep single-lane atomics as written: the wave-aggregating rewrite makes
    # the ticket draw wait for every load issued before it.
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip into libscan.so; returns its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-I", INCLUDE, "-I", CSRC, "-o", tmp] + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        subprocess.run(cmd, check=True)
    except BaseException:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
