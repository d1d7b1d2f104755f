"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The whole library is rebuilt with the sanitizers on its host side only (every
-fsanitize flag behind -Xarch_host; the device code is compiled as usual):
argument checks and launchers, the table codec and validator, split and
workspace sizing, the RoPE frequency tables and the block pool manager, all
driven through raw ctypes arrays.  The pool-manager and host-ABI tests then run
against that build in a child process with the sanitizer runtime preloaded;
any report fails the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "position_agnostic_kv_pool_amd", "csrc")
SOURCES = ["lazyattn_kernels.hip", "lazyattn_host.cpp", "lazyattn_pool.cpp", "lazyattn_runs.cpp"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def build_host_sanitized(out_path: str) -> None:
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    cmd += [os.path.join(CSRC, s) for s in SOURCES] + ["-o", out_path]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr[-4000:]


@pytest.mark.skipif(_hipcc() is None or _asan_runtime() is None, reason="hipcc or the clang ASan runtime missing")
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "liblazyattn_hostsan.so")
    build_host_sanitized(lib)
    log = str(tmp_path / "sanitizer")
    env = dict(os.environ,
               LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=1:log_path={log}",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={log}",
               LAZYATTN_LIBRARY=lib)
    tests = [os.path.join(ROOT, "tests", t) for t in ("test_pool.py", "test_abi_host.py")]
    proc = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
                          + tests, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = "".join(open(p).read() for p in glob.glob(log + "*"))
    assert reports == "", reports[:4000]
    assert proc.returncode == 0, (proc.stdout + proc.stderr)[-4000:]
    assert " passed" in proc.stdout
