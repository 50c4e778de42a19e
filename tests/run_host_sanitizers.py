"""Host AddressSanitizer + UndefinedBehaviorSanitizer run of the CPU test suite.

Builds two instrumented libraries under ``_build/sanitize/`` and runs the CPU tests against them in
subprocesses, each with the matching sanitizer runtime preloaded into Python:

1. the C oracle (``oracle/nvfp4_oracle.c``) with gcc ``-fsanitize=address,undefined``; the oracle
   tests run against it (``NVFP4_ORACLE_LIB``);
2. ``libnvfp4.so`` with the host side of every HIP source instrumented by clang
   (``-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined``; device code is not
   instrumented); the C-interface tests run against it (``NVFP4_LIB``): argument validation, status
   strings and the thread-local error text, all on the host.

Any sanitizer report aborts the process (``-fno-sanitize-recover``, ``halt_on_error``), which fails
the run. Usage: ``python tests/run_host_sanitizers.py`` (takes a few minutes, CPU only).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
sys.path.insert(0, ROOT)


def _runtime_clang() -> str:
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not hits:
        raise SystemExit("clang ASan runtime not found under /opt/rocm/llvm")
    return hits[0]


def _runtime_gcc(name: str) -> str:
    return subprocess.check_output(["gcc", f"-print-file-name={name}"], text=True).strip()


def build_oracle() -> str:
    import oracle
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "liboracle_san.so")
    flags = [f for f in oracle.CFLAGS if f != "-O2"] + ["-O1", "-g", "-fno-omit-frame-pointer",
                                                        "-fsanitize=address,undefined",
                                                        "-fno-sanitize-recover=all"]
    subprocess.check_call(["gcc", *flags, "-o", lib, oracle._SRC, "-lm"])
    return lib


def build_library() -> str:
    from nvfp4_w4a4_quantized_quantize_amd import build
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "libnvfp4_san.so")
    extra = ["-g", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-shared-libsan"]
    return build.build(extra=extra, out=lib)


def run(env_extra: dict, tests: list[str]) -> int:
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-m", "not gpu", "-p", "no:cacheprovider", *tests]
    print(" ".join(f"{k}={v}" for k, v in env_extra.items()), " ".join(cmd), flush=True)
    return subprocess.call(cmd, cwd=ROOT, env=env)


def main() -> int:
    oracle_lib = build_oracle()
    oracle_tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py"))) + \
        [os.path.join(ROOT, "tests", "test_sizes_and_workloads.py")]
    preload = f"{_runtime_gcc('libasan.so')}:{_runtime_gcc('libubsan.so')}"
    rc1 = run({"NVFP4_ORACLE_LIB": oracle_lib, "LD_PRELOAD": preload}, oracle_tests)
    lib = build_library()
    rc2 = run({"NVFP4_LIB": lib, "LD_PRELOAD": _runtime_clang()}, [os.path.join(ROOT, "tests", "test_abi_cpu.py")])
    print(f"oracle under gcc ASan+UBSan: rc={rc1}; C interface under clang ASan+UBSan: rc={rc2}", flush=True)
    return rc1 or rc2


if __name__ == "__main__":
    sys.exit(main())
