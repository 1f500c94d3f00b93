"""AddressSanitizer over the library's host code (beside the guard-band and determinism
checks, the memory checks of the library): the host side of csrc/flce_api.hip is compiled
with -fsanitize=address (the device code is built as usual and never run), and
tests/asan_host_check.c drives every size query, the planner, the host policy and the
argument checks that fail before any device call, with extreme and invalid arguments.
No GPU is used."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "chunked_lm_head_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


def test_host_code_is_clean_under_asan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm toolchain not found")
    lib = tmp_path / "libflce_asan.so"
    # the sanitizer on the host pass only: each -fsanitize= follows -Xarch_host, and the
    # device code (built, never run here) is not instrumented
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g",
                    "-std=c++17", "-fPIC", "-shared", "-Wno-unused-command-line-argument",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                    "-fno-omit-frame-pointer", "-fno-gpu-sanitize",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(CSRC, "flce_api.hip"), "-o", str(lib)], check=True)
    exe = tmp_path / "asan_host_check"
    subprocess.run([CLANG, "-std=c99", "-O1", "-g", "-fsanitize=address",
                    "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                    os.path.join(HERE, "asan_host_check.c"), str(lib),
                    f"-Wl,-rpath,{tmp_path}", "-o", str(exe)], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAIL" not in r.stdout, r.stdout
    assert "AddressSanitizer" not in r.stderr, r.stderr
    assert r.stdout.strip().startswith("ok "), r.stdout
