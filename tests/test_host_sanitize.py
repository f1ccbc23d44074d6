"""Host-side sanitizer run of the C ABI's validation and bookkeeping paths.

lcd_host.cpp (every check, the memory layout, split planning, the token counters and
checkpoint state) is built with the host C++ compiler under AddressSanitizer and
UndefinedBehaviorSanitizer, together with stand-ins for the HIP runtime and the kernel
launchers (tests/c/host_stubs.cpp), and driven through every entry point with valid and
invalid arguments by tests/c/host_validate.cpp.  No GPU and no HIP library is involved:
device pointers are fake addresses the host code must never dereference.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_decode_amd", "csrc")
HIP_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INCLUDE),
                    reason="needs g++ and the HIP headers")
def test_abi_host_paths_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_validate")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{HIP_INCLUDE}", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "lcd_host.cpp"), os.path.join(ROOT, "tests", "c", "host_stubs.cpp"),
           os.path.join(ROOT, "tests", "c", "host_validate.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert r.stdout.strip().splitlines()[-1].startswith("ok:"), r.stdout
