"""Build the HIP library libtq4.so in-tree for gfx950.

    python -m block_diffusion_lm_tq4_amd.build [--verbose]

Every translation unit is compiled by hipcc for gfx950 and linked into
``block_diffusion_lm_tq4_amd/libtq4.so``.  The encoder is compiled with
``-ffp-contract=off`` so that no product is fused into a sum in its fp64
arithmetic.  Packed fp32 vector instructions are switched off for all device
code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtq4.so")

SOURCES = {
    "codebook.cpp": [],
    "api.cpp": [],
    "pack.hip": ["-ffp-contract=off"],
    "rht.hip": [],
    "gemm.hip": [],
    "skinny.hip": [],
    "moe.hip": [],
    "probe.hip": [],
    "fp8.hip": ["-ffp-contract=off"],
}

ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm 7 is required to build libtq4.so)")


def _common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-fPIC",
        "-std=c++17",
        "-Wall",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link libtq4.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    common = _common_flags()

    def compile_one(item):
        src, extra = item
        obj = os.path.join(BUILD, src + ".o")
        cmd = [hipcc, *common, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd = [hipcc, "-x", "hip", *common, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        out = (res.stdout + res.stderr).strip()
        # hipcc's host pass does not know the packed-fp32 feature: harmless.
        lines = [ln for ln in out.splitlines()
                 if "packed-fp32-ops" not in ln and ln.strip()]
        if res.returncode != 0:
            raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{out}")
        if verbose and lines:
            print("\n".join(lines), file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=jobs or min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES.items()))

    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


SANITIZED_DIR = os.path.join(BUILD, "sanitized")
SANITIZED_LIB = os.path.join(SANITIZED_DIR, "libtq4.so")
# host-only sanitizers: each flag applies to the host pass of hipcc only, so
# device code is compiled exactly as in the normal build
_HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                  "-fno-omit-frame-pointer"]


def build_sanitized(verbose: bool = False) -> str:
    """libtq4.so with the host-side C-ABI layer (api.cpp, codebook.cpp) built
    under AddressSanitizer and UndefinedBehaviorSanitizer, the kernels as in
    the normal build; for running the ABI tests under the sanitizers (load it
    through TQ4_LIBRARY with the sanitizer runtime preloaded)."""
    hipcc = _hipcc()
    os.makedirs(SANITIZED_DIR, exist_ok=True)
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(SANITIZED_DIR, src + ".o")
        cmd = [hipcc, *_common_flags(), *extra]
        if src.endswith(".cpp"):
            cmd = [hipcc, "-x", "hip", *_common_flags(), *extra, *_HOST_SANITIZE]
        cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
        objs.append(obj)
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "lib", "llvm", "bin",
                         "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    cmd = [clang, "-shared", "-fPIC", "-fsanitize=address", "-fsanitize=undefined",
           "-shared-libsan", "-o", SANITIZED_LIB, *objs, "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    if verbose:
        print(f"built {SANITIZED_LIB}", file=sys.stderr)
    return SANITIZED_LIB


TEST_NATIVE = os.path.join(ROOT, "tests", "native")


def build_test_probes(verbose: bool = False) -> list[str]:
    """Compile the test-only kernels under tests/native/ (one shared library
    each, next to its source); returns their paths."""
    hipcc = _hipcc()
    out = []
    for src in sorted(os.listdir(TEST_NATIVE)) if os.path.isdir(TEST_NATIVE) else []:
        if not src.endswith(".hip"):
            continue
        lib = os.path.join(TEST_NATIVE, "lib" + src[:-4] + ".so")
        cmd = [hipcc, *_common_flags(), "-shared", os.path.join(TEST_NATIVE, src), "-o", lib]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
        if verbose:
            print(f"built {lib}", file=sys.stderr)
        out.append(lib)
    return out


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv)
    build_test_probes(verbose="--verbose" in sys.argv)
