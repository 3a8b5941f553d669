"""The C-ABI front end (argument validation, workspace sizes, status strings)
under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

attn_api.cpp is plain C++; it is compiled here with g++ -fsanitize=address,
undefined (no GPU code: the HIP launchers are replaced by host stubs that the
validation never reaches in these tests) into a shared library, and the whole
of tests/test_abi_cpu.py runs against it in a child process with the
sanitizer runtime preloaded.  Any report (out-of-bounds access, signed
overflow in a size computation, misaligned or invalid shift, ...) fails.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
API = os.path.join(ROOT, "exact_attention_121_amd", "csrc", "attn_api.cpp")
STUB = os.path.join(ROOT, "tests", "sanitize", "launch_stub.cpp")


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
@pytest.mark.skipif(bool(os.environ.get("LD_PRELOAD")), reason="another library is preloaded in this environment")
def test_abi_tests_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no libasan runtime")
    lib = tmp_path / "libattn_fwd_sanitized.so"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-shared", "-fPIC", API, STUB, "-o", str(lib)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ATTN_LIBRARY=str(lib), LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-m", "not gpu"],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
