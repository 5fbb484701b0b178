"""Build libpa.so (HIP kernels + C ABI) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libpa.so"
SOURCES = [CSRC / "pa_api.cpp", CSRC / "pa_block_manager.cpp", CSRC / "pa_workspace.cpp",
           CSRC / "pa_kernels.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags() -> list:
    return [
        "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
        # keep packed fp32 arithmetic out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        f"-I{ROOT / 'include'}", f"-I{CSRC}",
    ]


def build(verbose: bool = False) -> pathlib.Path:
    """Compile every source into libpa.so (always recompiles).  The sources
    are compiled to objects in parallel, then linked."""
    objdir = ROOT / "_build"
    objdir.mkdir(exist_ok=True)
    flags = [f for f in compile_flags() if f != "-shared"]
    jobs = []
    for src in SOURCES:
        obj = objdir / (src.name + ".o")
        cmd = [hipcc()] + flags + ["-c", str(src), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((cmd, obj, subprocess.Popen(cmd, cwd=str(PKG), stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
    failed = False
    for cmd, obj, proc in jobs:
        out, _ = proc.communicate()
        noise = [ln for ln in out.splitlines() if ln.strip() and "packed-fp32-ops" not in ln]
        if proc.returncode != 0:
            sys.stderr.write(out)
            failed = True
        elif verbose and noise:
            print("\n".join(noise), flush=True)
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared"] + \
        [str(o) for _, o, _ in jobs] + ["-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=str(PKG), capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc link failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
