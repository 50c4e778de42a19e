"""Build libnvfp4.so (hand-written HIP for gfx950) in-tree with hipcc.

Each HIP source is compiled to an object of its own, in parallel, and the objects are linked into
the shared library. The same run builds ``libnvfp4_selftest.so`` from ``csrc/selftest/``: device
checks of the library's own conversion and division helpers, loaded only by the test suite (the
product library neither contains nor exports them).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SELFTEST_SRC = os.path.join(CSRC, "selftest")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libnvfp4.so")
SELFTEST_LIB = os.path.join(PKG, "libnvfp4_selftest.so")
OBJDIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # packed FP32 instructions stay off (see the project's hardware notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def selftest_sources() -> list[str]:
    return sorted(glob.glob(os.path.join(SELFTEST_SRC, "*.hip")))


def _headers() -> list[str]:
    return glob.glob(os.path.join(CSRC, "*.h")) + [os.path.join(INCLUDE, "nvfp4.h")]


def digest(srcs: list[str]) -> str:
    """SHA-256 over the named sources, the package headers and the C interface header."""
    h = hashlib.sha256()
    for f in sorted(srcs) + sorted(_headers()):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed: {' '.join(cmd[-3:])}")


def _link(srcs: list[str], out: str, tag: str, extra: list[str], verbose: bool, jobs: int) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, f"{tag}_{os.path.splitext(os.path.basename(s))[0]}.o") for s in srcs]
    cmds = [[HIPCC, *FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = out + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    with open(out + ".digest", "w") as fh:
        fh.write(digest(srcs) + "\n")
    return out


def build(verbose: bool = False, jobs: int | None = None, extra: list[str] | None = None,
          out: str | None = None) -> str:
    """Compile libnvfp4.so (and the self-test module) for gfx950. ``extra`` adds hipcc flags (the
    host-sanitizer build passes ``-Xarch_host -fsanitize=...`` and its own ``out``)."""
    jobs = jobs or min(8, os.cpu_count() or 1)
    extra = list(extra or [])
    tag = "san" if extra else "rel"
    lib = _link(sources(), out or LIB, tag, extra, verbose, jobs)
    if out is None:
        _link(selftest_sources(), SELFTEST_LIB, "selftest", extra, verbose, jobs)
    return lib


def built_from_current_sources(lib: str, srcs: list[str]) -> bool:
    """True when ``lib`` exists and the digest written beside it at build time matches the sources
    as they are now (content, not modification times, so copies of the tree give the same answer)."""
    try:
        with open(lib + ".digest") as fh:
            return os.path.exists(lib) and fh.read().strip() == digest(srcs)
    except OSError:
        return False


def stale() -> bool:
    """True when libnvfp4.so or the self-test module is missing or was built from other sources."""
    return not (built_from_current_sources(LIB, sources()) and
                built_from_current_sources(SELFTEST_LIB, selftest_sources()))


if __name__ == "__main__":
    print(build(verbose=True))
