"""The C front end under AddressSanitizer and UBSan, on the CPU.

mha_api.cpp (argument validation, workspace arithmetic, status codes, the
thread-local error text) is built for the host with -fsanitize=address,undefined
and stub kernel launchers (tests/asan/launch_stubs.cpp), and the host ABI tests
are run against that library in a child process with the sanitizer runtime
preloaded: any out-of-bounds access, use after free or undefined behaviour on
those paths aborts the child. The one test that needs torch is left out.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _libasan():
    if shutil.which("g++") is None:
        return None
    path = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_libasan() is None or not os.path.exists("/opt/rocm/lib/libamdhip64.so"),
                    reason="needs g++ with libasan and the ROCm host runtime")
def test_front_end_under_address_sanitizer():
    sys.path.insert(0, ROOT)
    from transformer_scaled_dot_mha_amd import build
    lib = build.build_host_asan()
    env = dict(os.environ)
    env.update(MHA_LIBRARY=lib, LD_PRELOAD=_libasan(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    deselect = "not rejects_cpu_tensors"
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q",
                        "-p", "no:cacheprovider", "-k", deselect], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    passed = [ln for ln in out.splitlines() if " passed" in ln]
    assert passed and int(passed[-1].split(" passed")[0].split()[-1]) >= 90, out[-2000:]
