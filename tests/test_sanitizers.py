"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The C oracle (oracle/ckda_oracle.c) and the C-ABI library's host side
(api.cpp: argument, shape, alias and workspace validation) are rebuilt with
-fsanitize=address,undefined and driven through their existing host tests
(tests/test_oracle_pins.py, tests/test_abi.py) in a child process with the
sanitizer runtime preloaded; any report fails the test.  The GPU code is not
instrumented (the library's device objects are linked as built)."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _pytest(env, *args):
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider", *args],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isfile(asan):
        pytest.skip("gcc's AddressSanitizer runtime not found")
    lib = str(tmp_path / "libckda_oracle_san.so")
    subprocess.run([gcc, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    "-o", lib, os.path.join(ROOT, "oracle", "ckda_oracle.c"), "-lm"], check=True)
    env = dict(os.environ, CKDA_ORACLE_LIB=lib, LD_PRELOAD=asan, **SAN_ENV)
    out = _pytest(env, "tests/test_oracle_pins.py", "-m", "not gpu")
    assert "passed" in out


def test_host_validation_under_asan_and_ubsan(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = sorted(glob.glob(os.path.join(ROOT, "_build", "*.o")))
    objs = [o for o in objs if os.path.basename(o) != "api.o"]
    if not os.path.exists(hipcc) or not objs:
        pytest.skip("hipcc or the library's built objects (gated_delta_rule_sign_amd.build) are missing")
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rts:
        pytest.skip("clang's AddressSanitizer runtime not found")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    api_o = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libckda_san.so")
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san,
                    "-Xarch_host", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                    "-c", os.path.join(ROOT, "gated_delta_rule_sign_amd", "csrc", "api.cpp"), "-o", api_o],
                   check=True, capture_output=True)
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan", *san, "-o", lib, api_o, *objs],
                   check=True, capture_output=True)
    env = dict(os.environ, CKDA_LIB=lib, LD_PRELOAD=rts[0], **SAN_ENV)
    out = _pytest(env, "tests/test_abi.py")
    assert "passed" in out
