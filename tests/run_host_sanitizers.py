"""Host-code sanitizer run (AddressSanitizer + UndefinedBehaviorSanitizer), CPU only.

Builds, into _build/san/:
  * libnmspmv.so -- the C ABI (api.cpp) and every HIP source, the host side (argument
    checks, planners, launchers) compiled with the sanitizers (``-Xarch_host`` before each
    sanitizer flag: the device code is built as usual, without them); only the host
    tests load it, on a machine with or without a GPU;
  * libnmoracle.so -- the oracle's C code, with the same sanitizers;
then runs the host tests (``tests/test_abi_host.py`` and the oracle pin tests) against
those two libraries, with the clang sanitizer runtime preloaded into the Python process
(NM_SPMV_LIB / NM_ORACLE_LIB select the libraries).  Any sanitizer report aborts the
process (``-fno-sanitize-recover``, ``halt_on_error``), so the exit status is the verdict.

Usage: python tests/run_host_sanitizers.py [extra pytest args]
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "san")
CSRC = os.path.join(ROOT, "bitmask_spmv_amd", "csrc")
LLVM = "/opt/rocm/llvm"
HIPCC = "/opt/rocm/bin/hipcc"

SAN = ["address", "undefined"]
# each -fsanitize= directly after -Xarch_host: host pass only, never device code
HIP_SAN = [a for s in SAN for a in ("-Xarch_host", f"-fsanitize={s}")] + [
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
C_SAN = [f"-fsanitize={','.join(SAN)}", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
TESTS = ["tests/test_abi_host.py", "tests/test_oracle_pins.py", "tests/test_oracle_meta_pins.py",
         "tests/test_oracle_swiglu_pins.py", "tests/test_oracle_unstructured_pins.py"]


def runtime() -> str:
    libs = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not libs:
        raise FileNotFoundError("clang AddressSanitizer runtime (libclang_rt.asan-x86_64.so) not found under " + LLVM)
    return libs[-1]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def _stale(out: str, deps) -> bool:
    return not os.path.exists(out) or any(os.path.getmtime(d) > os.path.getmtime(out) for d in deps)


def build() -> tuple[str, str]:
    os.makedirs(OUT, exist_ok=True)
    headers = glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "api.cpp")]

    def comp(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        if _stale(obj, [src, *headers, __file__]):
            _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
                  f"-I{os.path.join(ROOT, 'include')}", "-x", "hip", "--offload-arch=gfx950",
                  *HIP_SAN, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(comp, srcs))
    lib = os.path.join(OUT, "libnmspmv.so")
    if _stale(lib, objs):
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HIP_SAN, "-Xarch_host", "-shared-libsan",
              "-o", lib, *objs])
    osrc = os.path.join(ROOT, "oracle", "nm_oracle.c")
    olib = os.path.join(OUT, "libnmoracle.so")
    if _stale(olib, [osrc, __file__]):
        # the oracle's own flags (strict IEEE fp64), plus the sanitizers
        _run([os.path.join(LLVM, "bin", "clang"), "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
              "-fPIC", "-shared", "-shared-libsan", "-pthread", "-Wall", "-Wextra", *C_SAN, "-o", olib, osrc, "-lm"])
    return lib, olib


def main(argv) -> int:
    lib, olib = build()
    env = dict(os.environ)
    env.update({
        "NM_SPMV_LIB": lib,
        "NM_ORACLE_LIB": olib,
        "LD_PRELOAD": runtime(),
        # Python itself is not instrumented: leak reports would be its own allocations
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1:exitcode=87",
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *TESTS, *argv]
    print("[sanitizers]", lib, olib, flush=True)
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
