"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

fa_api.cpp (argument validation, parameter set-up, dispatch) is compiled with g++ and
-fsanitize=address,undefined into a host-only library whose kernel launchers are stubs
(tests/c_abi/fa_launch_stubs.cpp: they check the launch parameters and count calls, and
touch no memory). tests/test_abi.py then runs against that library in a child process
with the ASan runtime preloaded: every rejection case, and valid calls up to the stated
size limits that reach the launchers, with any out-of-bounds access, overflow or other
undefined behaviour on the way aborting the run."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_tiled_attention_05_amd", "csrc")


def _runtime(name):
    try:
        path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                              timeout=30).stdout.strip()
    except (OSError, subprocess.SubprocessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None or _runtime("libasan.so") is None,
                    reason="g++ with the AddressSanitizer runtime is needed")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "libfa_host_sanitized.so"
    build = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared", "-fPIC",
             "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}",
             f"-I{CSRC}", os.path.join(CSRC, "fa_api.cpp"),
             os.path.join(ROOT, "tests", "c_abi", "fa_launch_stubs.cpp"), "-o", str(lib)]
    r = subprocess.run(build, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, FA_ABI_TEST_LIB=str(lib), LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    tail = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "failed" not in r.stdout, tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail
