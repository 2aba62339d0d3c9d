"""Build libqlora.so (gfx950) in-tree with hipcc.

Usage: python parameter_efficient_fine_nf4_amd/build.py [--verbose] [--sanitize]
(run as a file: importing the package needs the library this script builds)

Every source under csrc/ is compiled for gfx950 only, in parallel, and the
objects are linked into parameter_efficient_fine_nf4_amd/libqlora.so.  The
build always recompiles (it is the "does it build" check as well).

--sanitize builds a second copy, _build/asan/libqlora.so, whose HOST code
(argument validation, workspace carving, launch set-up) carries
AddressSanitizer and UndefinedBehaviorSanitizer; the device code is built
as usual.  It is for the host-only tests, run as

  LD_PRELOAD=$(hipcc --print-file-name=libclang_rt.asan-x86_64.so) \
  ASAN_OPTIONS=detect_leaks=0 QLORA_LIB_PATH=_build/asan/libqlora.so \
  python -m pytest tests/test_capi_host.py
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqlora.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["capi.hip", "timing.hip", "quant.hip", "merge.hip", "lora.hip", "gemm_fwd.hip", "gemm_dx.hip",
           "optim.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no implicit multiply-add contraction (hipcc's default contracts across
    # statements and ignores `#pragma clang fp contract`): the storage
    # format's block constant is two separately rounded fp32 operations
    "-ffp-contract=off",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-result",
]


# Host-side sanitizers only: each -fsanitize= applies to the host pass.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def _compile(src: str, verbose: bool, out_dir: str = OUT_DIR, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if verbose and msg:
        print(msg, flush=True)
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out_dir = os.path.join(OUT_DIR, "asan") if sanitize else OUT_DIR
    lib = os.path.join(out_dir, "libqlora.so") if sanitize else LIB
    extra = SANITIZE if sanitize else []
    os.makedirs(out_dir, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, out_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, "-shared-libsan", "-o", tmp, *objs] \
        if sanitize else [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    if not sanitize:
        import ctypes
        ctypes.CDLL(tmp)  # fails if any symbol (e.g. a kernel stub) is unresolved
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv, sanitize="--sanitize" in sys.argv))
