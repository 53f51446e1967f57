"""Build the gfx950 attention library ``libfa_mi355x.so`` in-tree with hipcc.

Each HIP source is compiled to an object in ``_build/`` (in parallel), then
linked into a shared library next to this file.  Flags: gfx950 only, -O3,
and the packed-fp32 VALU forms disabled (``-target-feature -packed-fp32-ops``);
the forward is scheduled with the compiler's iterative-ILP strategy and the
block's GEMMs with its max-ILP strategy, which measured faster there than the
default (and slower on the decode kernels, which keep the default).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfa_mi355x.so")
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip", "fa_kvcache.hip", "fa_block.hip",
           "fa_pager.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]
FILE_FLAGS = {"fa_fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
              "fa_block.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def flags_for(src: str) -> list:
    """The full hipcc flag list one source is compiled with."""
    return [*CFLAGS, *FILE_FLAGS.get(src, [])]


def _deps():
    out = [os.path.join(CSRC, f) for f in os.listdir(CSRC)]
    out.append(os.path.join(INCLUDE, "fa.h"))
    return out


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in _deps())


def build(force: bool = True, verbose: bool = False, extra_flags=(), lib: str = LIB, build_dir: str = BUILD_DIR,
          link_flags=()) -> str:
    """Compile every source and link ``lib``; ``extra_flags`` are added to each
    compile line and ``link_flags`` to the link line (the host-sanitizer build
    passes both and its own output paths)."""
    if not force and lib == LIB and not is_stale():
        return LIB
    os.makedirs(build_dir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *flags_for(src), *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the gfx feature flag; that note is harmless
        lines = [ln for ln in text.splitlines() if "not a recognized feature" not in ln]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for " + ", ".join(failed))
    tmp = lib + ".tmp"
    subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, *link_flags, "-o", tmp],
                   check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(force="--if-stale" not in sys.argv, verbose="-v" in sys.argv))
