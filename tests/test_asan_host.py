"""AddressSanitizer runs of the host code (CPU only, no GPU needed):

  * the C ABI's host-side validation: ``api.cpp`` compiled with host AddressSanitizer and linked with
    the regular build's kernel objects into ``_build/asan/libssd_asan.so``; ``tests/test_abi.py``
    (every entry point's argument checks, workspace queries, the export list) runs against it;
  * the fp64 oracle: ``oracle/ssd_oracle.c`` compiled by clang with AddressSanitizer; the oracle's
    pins (``tests/test_oracle*.py``) run against it.

Each run is a child pytest process with clang's AddressSanitizer runtime preloaded (leak checking
off: the interpreter itself is not instrumented) and must end cleanly with no sanitizer report.
Skipped where ROCm's clang, its AddressSanitizer runtime or the regular build's objects are missing.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_DIR = os.path.join(ROOT, "_build", "asan")
CSRC = os.path.join(ROOT, "selective_state_space_diag_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
KERNEL_OBJECTS = ["scan1", "conv1d", "selective", "hgrn2", "hgrn2_sweep", "norm"]
HOST_ASAN = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def _runtime():
    paths = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return paths[-1] if paths else None


def _objects():
    return [os.path.join(ROOT, "_build", n + ".o") for n in KERNEL_OBJECTS]


def _missing():
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG) and _runtime()):
        return "ROCm clang or its AddressSanitizer runtime is missing"
    if not all(os.path.exists(o) for o in _objects()):
        return "the regular build's objects are missing (run the library build first)"
    return None


pytestmark = pytest.mark.skipif(_missing() is not None, reason=str(_missing()))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-4000:]}"


def _build_library():
    os.makedirs(ASAN_DIR, exist_ok=True)
    obj = os.path.join(ASAN_DIR, "api_asan.o")
    lib = os.path.join(ASAN_DIR, "libssd_asan.so")
    _run([HIPCC, "-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950", *HOST_ASAN,
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, "api.cpp"), "-o", obj])
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-o", lib, obj,
          *_objects()])
    return lib


def _build_oracle():
    os.makedirs(ASAN_DIR, exist_ok=True)
    lib = os.path.join(ASAN_DIR, "liboracle_asan.so")
    _run([CLANG, "-std=c99", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-fPIC", "-shared",
          "-o", lib, os.path.join(ROOT, "oracle", "ssd_oracle.c"), "-lm"])
    return lib


def _child_pytest(env_extra, files):
    env = dict(os.environ, LD_PRELOAD=_runtime(), ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-m", "not gpu", "-p", "no:cacheprovider", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr, out
    assert " passed" in r.stdout, out


def _instrumented(lib):
    r = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True)
    return "__asan_report_load" in r.stdout


def test_abi_validation_under_address_sanitizer():
    lib = _build_library()
    assert _instrumented(lib)
    _child_pytest({"SSD_LIBRARY": lib}, ["tests/test_abi.py"])


def test_oracle_under_address_sanitizer():
    lib = _build_oracle()
    assert _instrumented(lib)
    _child_pytest({"SSD_ORACLE_LIBRARY": lib},
                  ["tests/test_oracle.py", "tests/test_oracle_block.py", "tests/test_oracle_variants.py",
                   "tests/test_oracle_grad.py"])
