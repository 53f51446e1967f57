"""Run the CPU test suite against host-sanitized builds (AddressSanitizer +
UndefinedBehaviorSanitizer) of the library's host code and of the oracle.

    python tests/run_sanitized.py [extra pytest args]

Builds into ``_build/san/``:
- the attention library, each source compiled as the product is, with the
  sanitizers on the host pass only (every ``-fsanitize=`` follows
  ``-Xarch_host``; the gfx950 device code is built exactly as in the product);
- the oracle, built with the same clang so that one sanitizer runtime serves
  both libraries in one process.

Then runs ``pytest -m "not gpu"`` on the tests that call into either library,
with the clang ASan runtime preloaded (the Python interpreter itself is not
instrumented), ``FA_MI355X_LIB`` and ``ORACLE_LIB`` pointing at the sanitized
builds, and every finding fatal.  Leak checking is off: the interpreter and
torch keep allocations alive until exit by design.  CPU only; nothing here
touches a GPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from flashattention_forward_03_amd import build as fa_build  # noqa: E402
from oracle import build as oracle_build  # noqa: E402

SAN_DIR = os.path.join(ROOT, "_build", "san")
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
TESTS = ["tests/test_abi.py", "tests/test_pager.py", "tests/test_oracle.py", "tests/test_oracle_block.py",
         "tests/test_inputs.py", "tests/test_bench.py"]


def asan_runtime() -> str:
    out = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], check=True,
                         capture_output=True, text=True).stdout.strip()
    if not os.path.isfile(out):
        raise RuntimeError(f"clang's ASan runtime not found (clang printed {out!r})")
    return out


def build_all() -> tuple:
    lib = fa_build.build(force=True, extra_flags=HOST_SAN, lib=os.path.join(SAN_DIR, "libfa_mi355x_san.so"),
                         build_dir=SAN_DIR, link_flags=["-Xarch_host", "-shared-libsan", *HOST_SAN[:2]])
    # the oracle through clang (host code only: no device pass to steer)
    orc = oracle_build.build(force=True, lib=os.path.join(SAN_DIR, "liboracle_san.so"),
                             extra_flags=["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                                          "-fno-omit-frame-pointer", "-g", "-shared-libsan"], cc=CLANG)
    return lib, orc


def main(argv) -> int:
    lib, orc = build_all()
    env = dict(os.environ)
    env.update({
        "FA_MI355X_LIB": lib,
        "ORACLE_LIB": orc,
        "LD_PRELOAD": asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    # the tests must load the sanitized builds, with the runtime active
    probe = ("import ctypes, flashattention_forward_03_amd as fa, oracle; fa.load_library(); oracle._load(); "
             "maps = open('/proc/self/maps').read(); "
             f"assert {lib!r} in maps and {orc!r} in maps, 'sanitized libraries not loaded'; "
             "assert hasattr(ctypes.CDLL(None), '__asan_init'), 'ASan runtime not active'")
    subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, check=True)
    cmd = [sys.executable, "-m", "pytest", *TESTS, "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *argv]
    print("+", " ".join(cmd), flush=True)
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
