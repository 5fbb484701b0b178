"""CPU: the library's host code built with AddressSanitizer and
UndefinedBehaviorSanitizer, with the block-manager and C-ABI suites run
against that build in a subprocess.

Host code: pa_api.cpp (argument checks, pa_check_inputs_host, the swap
bookkeeping), pa_block_manager.cpp (free sets, maps, reference counts) and
pa_workspace.cpp (the workspace layout), compiled by g++ with the sanitizers.
The kernels' object from the regular build is linked in uninstrumented: no
GPU code is sanitized, and no test here reaches a kernel launch.

By hand, from the repository root:

    python -c "from tests.test_host_sanitizers import build_sanitized as b; print(b())"
    LD_PRELOAD=$(g++ -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \\
        PA_LIBRARY=_build/san/libpa_san.so \\
        python -m pytest tests/test_block_manager.py tests/test_abi.py
"""
from __future__ import annotations

import os
import pathlib
import shutil
import subprocess
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
CSRC = ROOT / "paged_kv_cache_438_amd" / "csrc"
OUT = ROOT / "_build" / "san"
HOST_SOURCES = ["pa_api.cpp", "pa_block_manager.cpp", "pa_workspace.cpp"]
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer", "-g", "-O1"]


def _kernels_object() -> pathlib.Path:
    """The regular build's object of the kernel source, rebuilt if stale."""
    obj = ROOT / "_build" / "pa_kernels.hip.o"
    src = CSRC / "pa_kernels.hip"
    if not obj.exists() or obj.stat().st_mtime < max(src.stat().st_mtime,
                                                     (CSRC / "pa_launch.h").stat().st_mtime):
        from paged_kv_cache_438_amd.build import build
        build()
    return obj


def build_sanitized() -> pathlib.Path:
    """Compile the host sources with the sanitizers (g++) and link them with
    the kernels' object into _build/san/libpa_san.so."""
    OUT.mkdir(parents=True, exist_ok=True)
    objs = []
    for name in HOST_SOURCES:
        obj = OUT / (name + ".o")
        subprocess.run(["g++", "-std=c++17", "-fPIC", *SANITIZE, "-D__HIP_PLATFORM_AMD__",
                        "-I/opt/rocm/include", f"-I{ROOT / 'include'}", f"-I{CSRC}", "-c",
                        str(CSRC / name), "-o", str(obj)], check=True)
        objs.append(str(obj))
    lib = OUT / "libpa_san.so"
    subprocess.run(["g++", "-shared", "-fPIC", *SANITIZE, *objs, str(_kernels_object()),
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(lib)],
                   check=True)
    return lib


def _asan_runtime() -> str:
    r = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True)
    return r.stdout.strip()


needs_toolchain = pytest.mark.skipif(
    shutil.which("g++") is None or not os.path.exists("/opt/rocm/lib/libamdhip64.so"),
    reason="needs g++ with libasan and the HIP runtime library")


@needs_toolchain
@pytest.mark.timeout(900)
def test_host_code_under_address_and_ub_sanitizers():
    lib = build_sanitized()
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), PA_LIBRARY=str(lib),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the instrumented build and the sanitizer runtime are what gets loaded
    probe = subprocess.run(
        [sys.executable, "-c", "import paged_kv_cache_438_amd as pa; pa.load(); "
         "print(open('/proc/self/maps').read())"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-3000:]
    assert "libpa_san.so" in probe.stdout and "libasan" in probe.stdout
    assert "paged_kv_cache_438_amd/libpa.so" not in probe.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_block_manager.py", "tests/test_abi.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=800)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-5000:]
    assert r.returncode == 0, out[-5000:]
    assert " passed" in r.stdout and "failed" not in r.stdout
