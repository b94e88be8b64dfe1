"""The host side of the library (argument validation, planning, error strings) under
AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library is rebuilt with the sanitizers on its host code (device code is compiled as
usual) and the ABI tests, which drive every entry point's validation through ctypes, run
against that build in a child process with the ASan runtime preloaded. Any sanitizer
report ends the child with an error.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _asan_runtime():
    hits = sorted(glob.glob(os.path.join(ROCM, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def test_abi_validation_under_asan_and_ubsan(tmp_path):
    from bidirectional_transformer_attention_amd import build
    rt = _asan_runtime()
    if rt is None or not os.path.exists(build.HIPCC):
        pytest.skip("no hipcc or ASan runtime")
    lib = str(tmp_path / "libnxattn_host_san.so")
    # host code only: each sanitizer flag is scoped to the host compilation
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    build.build(verbose=False, out=lib, build_dir=str(tmp_path / "obj"), extra=san)
    env = dict(os.environ, LD_PRELOAD=rt, NXATTN_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child maps the sanitizer runtime and the sanitized build
    probe = subprocess.run([sys.executable, "-c", "import ctypes, os, sys; ctypes.CDLL(os.environ['NXATTN_LIBRARY']);"
                            "m = open('/proc/self/maps').read(); sys.exit(0 if 'asan' in m and "
                            "os.environ['NXATTN_LIBRARY'] in m else 3)"], env=env, capture_output=True, text=True)
    assert probe.returncode == 0, probe.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True, text=True)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
