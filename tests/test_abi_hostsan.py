"""The C ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

abi.cpp (argument validation, launch planning, workspace sizing) and plans.cpp are built host-only
with clang and both sanitizers, the kernel launchers replaced by stand-ins that launch nothing
(tests/hostsan/stubs.cpp), and tests/test_abi.py runs against that build in a child process with
the sanitizer runtime preloaded: every entry point's valid and invalid argument paths, with any
sanitizer report failing the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
CSRC = os.path.join(ROOT, "rank_kv_cache_lowrank_amd", "csrc")


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(not os.path.exists(CLANG) or _asan_runtime() is None, reason="clang or its ASan runtime missing")
def test_abi_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    so = str(tmp_path / "liblowrank_attn_hostsan.so")
    cmd = [CLANG, "-std=c++17", "-x", "c++", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libasan",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "plans.cpp"),
           os.path.join(ROOT, "tests", "hostsan", "stubs.cpp"), "-o", so]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), LOWRANK_ATTN_LIB=so,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout, out
