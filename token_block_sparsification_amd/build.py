"""Compile the HIP sources under csrc/ into libuniprefill.so (in-tree, gfx950).

Usage: python -m token_block_sparsification_amd.build [-v]
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libuniprefill.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU ops are disabled for every device function.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Wno-unused-variable", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return out


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer: every -fsanitize is
# preceded by -Xarch_host, so only the host code (argument checks, workspace
# layouts, chunk rules, launch set-up) is instrumented; device code is built
# as usual.  The library then needs the clang ASan runtime (which also holds
# the UBSan handlers) loaded first, e.g. LD_PRELOAD.
HOST_SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]


def asan_runtime() -> str:
    """Path of the clang ASan runtime matching hipcc's clang."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    return subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                          stdout=subprocess.PIPE, text=True, check=True).stdout.strip()


def build(verbose: bool = False, jobs: int = 4, out: str = LIB, objdir: str = OBJDIR,
          host_sanitize: bool = False) -> str:
    """Compile every csrc/*.hip and link the library `out`; returns its path.
    host_sanitize: instrument the host code with ASan + UBSan (see above)."""
    os.makedirs(objdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    flags = HIP_FLAGS + (HOST_SANITIZE_FLAGS if host_sanitize else [])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, [HIPCC, *flags, "-c", s, "-o", o], verbose)
                for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
