"""Build libpkv.so (host pool + gfx950 HIP kernels) in-tree with hipcc.

    python -m paged_kv_cache_pkv_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpkv.so")
PROBE_LIB = os.path.join(HERE, "libpkv_probe.so")  # bandwidth probes: a measurement aid, not the product ABI
OBJDIR = os.path.join(ROOT, "_build", "obj")

SOURCES = ["errors.cpp", "pool.cpp", "append.hip", "decode.hip", "prefill.hip", "blocks.hip", "fp8.hip", "prefix.hip", "check.hip"]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]
# Packed fp32 VALU forms are kept out of the generated code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if ln.strip() and noise not in ln]
    if msgs and verbose:
        print("\n".join(msgs), flush=True)


def _link(cc, sources, lib, verbose):
    objs = []
    for src in sources:
        path = os.path.join(CSRC, src)
        obj = os.path.join(OBJDIR, src + ".o")
        lang = ["-x", "hip"] + DEVICE if src.endswith(".hip") else ["-x", "c++"]
        _run([cc, *COMMON, *lang, "-c", path, "-o", obj], verbose)
        objs.append(obj)
    tmp = lib + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source (always) and link libpkv.so, and the bandwidth
    probes into libpkv_probe.so; returns libpkv.so's path."""
    os.makedirs(OBJDIR, exist_ok=True)
    cc = hipcc()
    _link(cc, SOURCES, LIB, verbose)
    _link(cc, ["probe.hip"], PROBE_LIB, verbose)
    return LIB


POOL_SANITIZED = os.path.join(ROOT, "_build", "libpkv_pool_sanitized.so")


def build_pool_sanitized(verbose: bool = False) -> str:
    """The host block pool alone (pool.cpp, errors.cpp), built with g++ under
    AddressSanitizer and UndefinedBehaviorSanitizer into a test-only library.
    It holds the pool's symbols and no device code; tests load it into a
    process that preloads the sanitizer runtimes."""
    os.makedirs(os.path.dirname(POOL_SANITIZED), exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in ("errors.cpp", "pool.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", f"-I{INCLUDE}", f"-I{CSRC}", *srcs,
           "-o", POOL_SANITIZED + ".tmp"]
    _run(cmd, verbose)
    os.replace(POOL_SANITIZED + ".tmp", POOL_SANITIZED)
    return POOL_SANITIZED


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
