"""The host side of the C ABI under AddressSanitizer (CPU only, no launch).

libpolar is built once more with AddressSanitizer on its host code only (every
``-fsanitize=`` behind ``-Xarch_host``; device code is built as usual and never runs
here), and tests/test_abi.py runs again in a child process against that build, with the
sanitizer's runtime preloaded: every argument check, error path, workspace-size function
and status string then runs under the sanitizer, and any heap or stack misuse in them
ends the child with a report.  Skipped where the toolchain's runtime is missing."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from long_context_lm_amd import build as libbuild  # noqa: E402

RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))


@pytest.mark.skipif(not RUNTIME or not os.path.exists(libbuild.HIPCC),
                    reason="no hipcc or AddressSanitizer runtime")
def test_abi_checks_under_address_sanitizer(tmp_path):
    out = str(tmp_path / "libpolar_asan.so")
    flags = [f for f in libbuild.FLAGS if f != "-O3"]
    cmd = [libbuild.HIPCC, "-O1", "-g", *flags, "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
           *[os.path.join(libbuild.CSRC, s) for s in libbuild.SOURCES], "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, LD_PRELOAD=RUNTIME[-1], POLAR_TEST_LIBRARY=out,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    tail = (run.stdout + run.stderr)[-4000:]
    assert run.returncode == 0, tail
    assert "AddressSanitizer" not in run.stderr, tail
    assert " passed" in run.stdout, tail
    assert f"[abi] library {out}" in run.stdout, tail        # the child ran the ASan build
