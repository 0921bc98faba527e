"""Sanitizer builds of the host code (CPU): the C oracle, and the host side of the
C ABI library, each built with AddressSanitizer and UndefinedBehaviorSanitizer and
driven by a small C program (tests/sanitize_*_main.c) on valid and invalid
arguments.  A sanitizer report aborts the driver, which fails the test.  The GPU code
of the library is built as usual (the sanitizers apply to host code only)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "san_oracle")
    _run(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wno-unknown-pragmas",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          os.path.join(HERE, "sanitize_oracle_main.c"), os.path.join(ROOT, "oracle", "moe_ref.c"),
          "-o", exe, "-lm"])
    assert "oracle sanitizer run ok" in _run([exe], env=ENV)


def test_abi_host_side_under_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from routed_int4_expert_amd import build as B
    clang = os.path.join(os.path.dirname(os.path.realpath(B.HIPCC)), "..", "lib", "llvm", "bin", "clang")
    if not (os.path.exists(B.HIPCC) and os.path.exists(clang)):
        pytest.skip("the ROCm toolchain is not installed")
    lib = str(tmp_path / "libmoe_san.so")
    san = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    B.build(extra=san, out=lib)
    exe = str(tmp_path / "san_abi")
    _run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(HERE, "sanitize_abi_main.c"), lib, "-Wl,-rpath," + str(tmp_path), "-o", exe])
    try:
        import torch
        gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        gpu = False
    out = _run([exe] + ([] if gpu else ["nogpu"]), env=ENV)
    assert "abi sanitizer run ok" in out
