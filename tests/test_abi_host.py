"""The host side of the boundary, on the CPU: libcsa's validation layer refuses invalid calls
before any launch (tests/abi_host_driver.cpp), its full validation plus workspace carving of a
decode step costs well under a microsecond per call ("TileLang, and a theorem prover in the
compiler": host-side contract checks in compiled code, under a microsecond), and the same cases
run clean under AddressSanitizer and UndefinedBehaviorSanitizer (host code of api.hip built with
them; device code untouched)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_long_context_csa_amd")
LIB = os.path.join(PKG, "libcsa.so")
DRIVER = os.path.join(ROOT, "tests", "abi_host_driver.cpp")
OUT = os.path.join(ROOT, "_build", "host_checks")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang++"


def _run(cmd, env=None, timeout=600):
    p = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return p.returncode, p.stdout + p.stderr


def _need(path):
    if not os.path.exists(path):
        pytest.skip(f"{path} not available")


def test_host_validation_cost_under_a_microsecond():
    _need(LIB)
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "abi_host_driver")
    rc, log = _run(["g++", "-O2", "-std=c++17", f"-I{ROOT}/include", DRIVER, "-o", exe,
                    f"-L{PKG}", "-lcsa", f"-Wl,-rpath,{PKG}"])
    assert rc == 0, log
    rc, log = _run([exe, "200000"])
    assert rc == 0 and "ok" in log, log
    ns = float(log.split("validate_ns_per_call")[1].split()[0])
    print(f"csa_decode_step host validation + workspace carving: {ns:.1f} ns per call")
    assert ns < 1000.0, log


def test_host_validation_under_asan_ubsan():
    _need(HIPCC)
    _need(CLANG)
    objs = [os.path.join(ROOT, "_build", f.replace(".hip", ".o"))
            for f in os.listdir(os.path.join(PKG, "csrc")) if f.endswith(".hip") and f != "api.hip"]
    for o in objs:
        _need(o)
    os.makedirs(OUT, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
    api_o = os.path.join(OUT, "api_san.o")
    rc, log = _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-Wno-unused-command-line-argument", f"-I{ROOT}/include",
                    f"-I{PKG}/csrc", *san, "-c", os.path.join(PKG, "csrc", "api.hip"),
                    "-o", api_o])
    assert rc == 0, log
    lib = os.path.join(OUT, "libcsa_san.so")
    rc, log = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, api_o, *objs])
    assert rc == 0, log
    exe = os.path.join(OUT, "abi_host_driver_san")
    rc, log = _run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", f"-I{ROOT}/include", DRIVER, "-o", exe, lib,
                    f"-Wl,-rpath,{OUT}"])
    assert rc == 0, log
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    rc, log = _run([exe, "2000"], env=env)
    assert rc == 0 and "ok" in log, log
    assert "AddressSanitizer" not in log and "runtime error" not in log, log
