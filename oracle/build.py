"""Compile the fp64 oracle (test infrastructure) into ``oracle/liboracle.so``.

Plain gcc, -O2, no fast-math: the oracle's arithmetic is IEEE double.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = True, lib: str = LIB, extra_flags=(), cc: str = "gcc") -> str:
    """Compile ``lib`` with ``cc``; ``extra_flags`` (the sanitizer build's) go on its line."""
    if not force and lib == LIB and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = lib + ".tmp"
    cmd = [cc, "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11", "-fPIC",
           "-shared", "-Wall", "-Wextra", *extra_flags, "-o", tmp, SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(force="--if-stale" not in sys.argv))
