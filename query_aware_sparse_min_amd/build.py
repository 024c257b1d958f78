"""Compile the HIP sources of the library into libsa.so for gfx950 (in-tree)."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libsa.so")
BUILD_DIR = os.path.join(ROOT, "_build", "sa")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are disabled for every kernel; default IEEE fp32
# division/sqrt and no fast-math, so encodings (int4 codes) are reproducible.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build: every sanitizer
# flag is for the host pass only (GPU code is never instrumented).
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, verbose: bool, build_dir: str, extra) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    # the host pass does not know the device-only feature flag: drop that warning
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise and verbose:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(verbose: bool = False, out: str = LIB, sanitize_host: bool = False) -> str:
    """Build libsa.so (in-tree by default); sanitize_host: host code instrumented with
    AddressSanitizer and UndefinedBehaviorSanitizer (load it with the clang ASan runtime
    preloaded)."""
    build_dir = BUILD_DIR + ("_host_asan" if sanitize_host else "")
    extra = HOST_SANITIZE if sanitize_host else []
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *extra, "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
