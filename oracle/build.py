"""Compile the C oracle into ``oracle/liboracle.so`` with gcc.

Test infrastructure: the oracle is the checker of the HIP library, never part
of it.  Called by ``__graft_entry__.build()`` and, when the shared object is
missing, by ``oracle.load()``.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Build liboracle.so from oracle.c; returns its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-O2", "-Wall", "-Wextra", "-Werror",
           "-fPIC", "-shared", "-pthread", "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
