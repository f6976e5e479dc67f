"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle (C, gcc) and the library's host code (hipcc; the sanitizer flags
apply to the host compilation only, device code is built as usual) are built
with ASan + UBSan into a temporary directory, and the tests that exercise them
without a GPU run in a child process with the matching sanitizer runtime
preloaded: the oracle pins, the residency pins, the residency policy parity
and the ABI checks.  Any sanitizer report aborts the child, which fails the
test."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hierarchical_sparse_kv_resolve_amd", "csrc")

pytestmark = pytest.mark.slow


def _run_child(preload, module, attr, lib, tests):
    code = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        f"import {module} as m\n"
        f"m.{attr} = {lib!r}\n"
        "import pytest\n"
        f"rc = pytest.main(['-q', '-x', '-p', 'no:cacheprovider', *{tests!r}])\n"
        f"assert {lib!r} in open('/proc/self/maps').read(), 'sanitized library not loaded'\n"
        "sys.exit(rc)\n")
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    assert p.returncode == 0, p.stdout[-3000:] + p.stderr[-3000:]


def test_oracle_under_asan_ubsan(tmp_path):
    runtime = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    if not os.path.isabs(runtime) or not os.path.exists(runtime):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liborc_san.so")
    subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-fPIC", "-shared", "-pthread",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "kvr_oracle.c"),
                    "-o", lib], check=True)
    _run_child(runtime, "oracle.oracle", "LIB_PATH", lib,
               ["tests/test_oracle_pins.py", "tests/test_residency_pins.py"])


def test_library_host_code_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc")
    runtimes = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not hipcc or not runtimes:
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "libkvr_san.so")
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-mcode-object-version=5", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *sorted(glob.glob(os.path.join(CSRC, "*.hip"))), "-o", lib]
    subprocess.run(cmd, check=True, capture_output=True, timeout=900)
    _run_child(runtimes[0], "hierarchical_sparse_kv_resolve_amd.kvr", "LIB_PATH", lib,
               ["tests/test_residency_policy.py", "tests/test_abi.py"])
