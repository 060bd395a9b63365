"""The C-ABI checks (tests/test_abi.py) against a build whose host-side layer
(argument validation, workspace layout, dispatch, codebook) runs under
AddressSanitizer and UndefinedBehaviorSanitizer.  No GPU is needed: every
call in those tests returns before any kernel launch, and any sanitizer
report aborts the child process."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def _stale(lib):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = [os.path.join(ROOT, "include", "tq4.h")]
    csrc = os.path.join(ROOT, "block_diffusion_lm_tq4_amd", "csrc")
    srcs += [os.path.join(csrc, f) for f in os.listdir(csrc)]
    return any(os.path.getmtime(s) > t for s in srcs)


def test_abi_checks_pass_under_asan_and_ubsan():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    sys.path.insert(0, ROOT)
    from block_diffusion_lm_tq4_amd import build as B
    lib = B.SANITIZED_LIB
    if _stale(lib):
        B.build_sanitized()
    runtime = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"],
                             capture_output=True, text=True).stdout.strip()
    assert os.path.exists(runtime), runtime
    env = dict(os.environ)
    env.update(TQ4_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out
