"""Build libdspark.so (the C-ABI HIP library) in-tree for gfx950.

    python semi_autoregressive_block_amd/build.py [--sanitized]

(run it by path: importing the package requires the built library)

Compiles every csrc/*.hip and csrc/*.cpp with hipcc (device code for gfx950
only, packed-FP32 instruction selection disabled) into objects under
_build/, in parallel, then links the shared library next to this file.
Always recompiles: a stale library is never trusted.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdspark.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    "-Wno-pass-failed", "-Wno-unused-result",
]


# Host-side checking build: the same sources with AddressSanitizer and
# UndefinedBehaviorSanitizer on the host code only (device code is built as
# usual); it is loaded only by the CPU tests of the argument validation.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
SAN_BUILD = os.path.join(BUILD, "sanitized")
SAN_LIB = os.path.join(SAN_BUILD, "libdspark_sanitized.so")


def _compile(src: str, sanitized: bool = False) -> str:
    out_dir = SAN_BUILD if sanitized else BUILD
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *(SANITIZE if sanitized else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines()
                     if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    return obj


def build(verbose: bool = False, sanitized: bool = False) -> str:
    out_dir, lib = (SAN_BUILD, SAN_LIB) if sanitized else (BUILD, LIB)
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    if not srcs:
        raise RuntimeError("no sources under " + CSRC)
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitized), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(SANITIZE if sanitized else []), "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources")
    return lib


if __name__ == "__main__":
    build(verbose=True, sanitized="--sanitized" in sys.argv[1:])
    sys.exit(0)
