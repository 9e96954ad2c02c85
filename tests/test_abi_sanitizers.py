"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

``vmla_api.cpp`` (validation, aliasing checks, RoPE table, launch arguments)
is compiled with g++ and both sanitizers, linked against counting launcher
stubs (``tests/sanitizer/launch_stubs.cpp``) instead of the gfx950 kernels,
and ``tests/test_abi.py`` runs against that build in a child process with the
ASan runtime preloaded. Any sanitizer report aborts the child, so the test
passes only if every check of test_abi.py passes and no report is printed.
The stub build also runs ``test_valid_calls_reach_the_launchers``, which
drives every entry point with valid arguments through to its launcher.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "latent_kv_attention_cache_amd", "csrc")


def test_host_abi_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    lib = str(tmp_path / "libvmla_host_sanitized.so")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}",
           f"-I{CSRC}", "-fPIC", "-shared", os.path.join(CSRC, "vmla_api.cpp"),
           os.path.join(ROOT, "tests", "sanitizer", "launch_stubs.cpp"), "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    assert os.path.isabs(asan) and os.path.exists(asan), asan
    env = dict(os.environ)
    # the ASan runtime must come first among the preloaded libraries
    env["LD_PRELOAD"] = ":".join(p for p in (asan, os.environ.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"   # the interpreter itself leaks by design
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["VMLA_LIBRARY"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-rs",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    # the stub-only test ran instead of being skipped
    assert "test_valid_calls_reach_the_launchers" not in out, out[-2000:]
