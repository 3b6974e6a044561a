"""CPU sanitizer tier: the host code under AddressSanitizer and UBSan.

Two instrumented builds go to _build/san/ and the CPU suites run against them
in child processes (the sanitizer runtime has to be loaded before Python's own
allocations, hence LD_PRELOAD in a fresh interpreter):

* libssmscan_san.so: the C-ABI front end (api.cpp, every host-side check of a
  call) and the launch log compiled with -fsanitize=address,undefined for the
  host only; the kernel objects are the regular build's. tests/test_abi_cpu.py
  runs against it through SSM_SCAN_LIBRARY. Those tests issue no device work.
* liboracle_san.so: the float64 oracle (ssm_oracle.c) with the same
  sanitizers; the oracle pin suites run against it through SSM_ORACLE_LIBRARY.

Errors are fatal (-fno-sanitize-recover=all), so any report fails the child
run. An instrumented library only loads when the sanitizer runtime is present,
so a passing run is a run under the sanitizers.

Run on its own with: python -m pytest tests/test_sanitizers_cpu.py -v
"""
import glob
import os
import shlex
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "selective_state_space_67_amd")
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(ROOT, "_build", "san")
HOST_SAN = shlex.split("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                       "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=86",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87"}
ORACLE_PINS = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*pins.py")))


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, "%s\n%s%s" % (" ".join(cmd), res.stdout[-4000:], res.stderr[-4000:])
    return res


def _regular_objects():
    """The regular build's objects (rebuilt when a source is newer)."""
    from selective_state_space_67_amd import build as bd

    objs = [os.path.join(bd.OBJ, os.path.splitext(s)[0] + ".o") for s in bd.SOURCES]
    newest_src = max(os.path.getmtime(p) for p in glob.glob(os.path.join(CSRC, "*")) +
                     [os.path.join(ROOT, "include", "ssm_scan.h")])
    if not all(os.path.exists(o) for o in objs) or min(os.path.getmtime(o) for o in objs) < newest_src:
        bd.build()
    return bd, objs


def _asan_runtime_clang():
    paths = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not paths:
        pytest.skip("clang AddressSanitizer runtime not found")
    return paths[-1]


def _nm_has_asan(path):
    res = _run(["nm", "-D", "--undefined-only", path])
    return "__asan_report" in res.stdout


@pytest.fixture(scope="module")
def san_library():
    bd, objs = _regular_objects()
    os.makedirs(OUT, exist_ok=True)
    common = [bd.hipcc(), "--offload-arch=" + bd.ARCH, "-O1", "-g", "-std=c++17", "-fPIC", "-Wall",
              "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, *bd.DEVICE_FLAGS, *HOST_SAN]
    san_objs = []
    for src in ("api.cpp", "log.cpp"):
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        _run(common + ["-c", "-o", obj, os.path.join(CSRC, src)])
        san_objs.append(obj)
    rest = [o for o in objs if os.path.basename(o) not in ("api.o", "log.o")]
    lib = os.path.join(OUT, "libssmscan_san.so")
    _run([bd.hipcc(), "--offload-arch=" + bd.ARCH, "-shared", "-fPIC", *HOST_SAN, "-shared-libsan", "-o", lib]
         + san_objs + rest)
    assert _nm_has_asan(lib)
    return lib


@pytest.fixture(scope="module")
def san_oracle():
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "liboracle_san.so")
    _run(["gcc", "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-std=c99", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", lib,
          os.path.join(ROOT, "oracle", "ssm_oracle.c"), "-lm"])
    assert _nm_has_asan(lib)
    return lib


def _pytest_child(files, env_extra, timeout):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + files
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    text = res.stdout + res.stderr
    assert "AddressSanitizer" not in text and "runtime error:" not in text, text[-6000:]
    assert res.returncode == 0, text[-6000:]
    return text


def test_abi_checks_under_asan_and_ubsan(san_library):
    text = _pytest_child([os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                         {"LD_PRELOAD": _asan_runtime_clang(), "SSM_SCAN_LIBRARY": san_library}, timeout=600)
    assert " passed" in text


def test_oracle_pins_under_asan_and_ubsan(san_oracle):
    libasan = _run(["gcc", "-print-file-name=libasan.so"]).stdout.strip()
    if not os.path.isabs(libasan):
        pytest.skip("gcc AddressSanitizer runtime not found")
    text = _pytest_child(ORACLE_PINS, {"LD_PRELOAD": libasan, "SSM_ORACLE_LIBRARY": san_oracle}, timeout=900)
    assert " passed" in text
