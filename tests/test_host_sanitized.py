"""The host side of the C ABI (argument validation, workspace sizing, error
texts, timing bookkeeping: gdr_api.hip and gdr_timing.hip) built for the
host with AddressSanitizer and UndefinedBehaviorSanitizer, and the ABI
validation tests re-run against it (CPU only; kernel launchers are stubs
that no validation test reaches)."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_chunk_amd", "csrc")


def _asan_runtime():
    base = "/opt/rocm/llvm/lib/clang"
    if not os.path.isdir(base):
        return None
    for ver in sorted(os.listdir(base), reverse=True):
        p = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def test_abi_validation_under_host_asan_and_ubsan():
    rt = _asan_runtime()
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if not rt or not os.path.exists(hipcc):
        pytest.skip("hipcc or the clang ASan runtime is not installed")
    with tempfile.TemporaryDirectory() as tmp:
        lib = os.path.join(tmp, "libgdr_hostsan.so")
        cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all",
               f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-o", lib,
               os.path.join(CSRC, "gdr_api.hip"), os.path.join(CSRC, "gdr_timing.hip"),
               os.path.join(ROOT, "tests", "host_launch_stub.hip")]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
        env = dict(os.environ, GDR_LIBRARY=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
        res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                              os.path.join(ROOT, "tests", "test_abi.py")],
                             cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        log = res.stdout + res.stderr
        assert "Sanitizer" not in log and "runtime error" not in log, log[-4000:]
        assert res.returncode == 0, log[-4000:]
        assert " passed" in res.stdout
