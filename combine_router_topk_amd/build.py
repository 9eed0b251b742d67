"""Builds libmoe_route.so (all HIP sources under csrc/) for gfx950 with hipcc.

Run `python combine_router_topk_amd/build.py` (by path: importing the package
loads the library) or call build() from a module loaded by path. Objects go to
_build/ at the repository root; the library lands next to this file. The module
imports nothing from the package.
"""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_route.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS_BASE = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
CFLAGS = CFLAGS_BASE + [f"-I{INCLUDE}", f"-I{CSRC}"]


def source_files() -> list[str]:
    """Every file the library is compiled from: the HIP sources and headers
    under csrc/ and the public header."""
    pats = [os.path.join(CSRC, "*.hip"), os.path.join(CSRC, "*.hpp"), os.path.join(INCLUDE, "*.h")]
    return sorted(f for p in pats for f in glob.glob(p))


def source_digest() -> str:
    """Build id: the first 16 hex digits of a SHA-256 over the compile flags
    and, in path order, each source file's path (relative to the repository)
    and bytes. The library returns the id it was built with from
    moe_build_id(), so a loader can tell a library built from other sources."""
    h = hashlib.sha256(" ".join(CFLAGS_BASE).encode())
    for f in source_files():
        h.update(b"\0" + os.path.relpath(f, ROOT).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out)


def build(jobs: int = 8) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(OBJDIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    bid = f'-DMOE_BUILD_ID="{source_digest()}"'
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _run([HIPCC, *CFLAGS, bid, "-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


C_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "check_abi.c")
C_CHECK_LIB = os.path.join(ROOT, "tests", "c_abi", "libcheck_abi.so")


def build_c_check() -> str:
    """The plain-C caller of the library used by the tests (gcc, C11): a
    shared library with moe_c_abi_check(), found by the tests next to its
    source; it finds libmoe_route.so through its run path."""
    tmp = C_CHECK_LIB + ".tmp"
    _run(["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
          "-I/opt/rocm/include", f"-I{INCLUDE}", C_CHECK_SRC, f"-L{PKG}", "-lmoe_route",
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../combine_router_topk_amd",
          "-Wl,-rpath,/opt/rocm/lib", "-o", tmp])
    os.replace(tmp, C_CHECK_LIB)
    return C_CHECK_LIB


if __name__ == "__main__":
    print(build())
    print(build_c_check())
