"""AddressSanitizer + UndefinedBehaviorSanitizer runs of the host code (CPU only).

Two builds into a temporary directory, each exercised by the existing CPU tests in
a child process with the matching sanitizer runtime preloaded:

* the C ABI's argument checks (sscan_capi.cpp) compiled with the host sanitizers
  and linked with the library's other objects; test_abi_cpu.py then drives every
  validate entry point, the workspace-size and plan queries and the spiral order
  through it, and test_abi_fuzz_cpu.py its randomised calls (no kernel is launched);
* the fp64 oracle's C sources built by gcc with the same sanitizers; the oracle
  pin tests then run on it.

Any report (out-of-bounds access, use after free, signed overflow, misaligned
load, ...) aborts the child and fails the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from selective_state_space_sscan_amd import build as B  # noqa: E402
from oracle import oracle  # noqa: E402

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run_tests(files, extra_env, tmp_path):
    # reports go to files (the child's pytest holds on to stderr)
    log = str(tmp_path / "sanitizer")
    env = dict(ENV, **extra_env)
    env["ASAN_OPTIONS"] += ":log_path=" + log
    env["UBSAN_OPTIONS"] += ":log_path=" + log
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + files
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = "".join(open(f).read()[:4000] for f in glob.glob(log + "*"))
    tail = "\n".join((r.stdout + r.stderr).splitlines()[-30:])
    assert r.returncode == 0 and not reports, reports + tail
    assert " passed" in tail, tail


def test_c_abi_checks_under_asan_ubsan(tmp_path):
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rts:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    objs = [os.path.join(B.OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "sscan_capi.cpp"]
    if not all(os.path.exists(o) for o in objs):
        B.build(force=False)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    capi = str(tmp_path / "sscan_capi.o")
    lib = str(tmp_path / "libsscan_asan.so")
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
              "-fvisibility=hidden", "-I", B.INCLUDE, "-I", B.CSRC]
    subprocess.run([B.hipcc()] + common + san + ["-c", "-o", capi, os.path.join(B.CSRC, "sscan_capi.cpp")],
                   check=True, capture_output=True)
    subprocess.run([B.hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + san + ["-o", lib, capi] + objs,
                   check=True, capture_output=True)
    _run_tests(["tests/test_abi_cpu.py", "tests/test_abi_fuzz_cpu.py"], {"SSCAN_TEST_LIBRARY": lib, "LD_PRELOAD": rts[0]},
               tmp_path)


def test_oracle_under_asan_ubsan(tmp_path):
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_asan.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    "-o", lib, *oracle.SOURCES, "-lm", "-lpthread"], check=True, capture_output=True)
    _run_tests(["tests/test_oracle_pins.py", "tests/test_oracle_bwd_pins.py", "tests/test_oracle_conv_pins.py",
                "tests/test_oracle_orders_pins.py", "tests/test_oracle_golden.py"],
               {"SSCAN_ORACLE_LIB": lib, "LD_PRELOAD": rt}, tmp_path)
