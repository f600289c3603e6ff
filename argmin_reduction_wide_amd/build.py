"""Build the gfx950 HIP library ``libargreduce.so`` in-tree with hipcc.

Usage: ``python -m argmin_reduction_wide_amd.build`` (also called by
``__graft_entry__.build()``). The library lands next to this file, where the Python
binding loads it from.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libargreduce.so")
SOURCES = [os.path.join(CSRC, "argreduce_kernels.hip"), os.path.join(CSRC, "argreduce_scan.hip"),
           os.path.join(CSRC, "argreduce_api.cpp")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def flags() -> list[str]:
    return [
        "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
        "-fvisibility=hidden", "-mcode-object-version=5",
        # IEEE comparisons with subnormals: no fast-math, no flush-to-zero.
        "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
        # no packed-fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # kernel arguments preloaded into SGPRs at wave launch (gfx950 supports it; the
        # code object keeps a loading prologue for firmware that does not)
        "-mllvm", "-amdgpu-kernarg-preload-count=16",
        "-I", INCLUDE, "-I", CSRC,
    ]


def fast_binding_path() -> str:
    import sysconfig

    return os.path.join(PKG, "_argreduce_fast" + sysconfig.get_config_var("EXT_SUFFIX"))


def build_fast_binding(verbose: bool = False) -> str:
    """Compile the CPython fast-call marshalling module (host C, no device code) next to the
    library; it links against the Python runtime only."""
    import sysconfig

    out = fast_binding_path()
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for the fast-call binding")
    cmd = [cc, "-O2", "-std=c11", "-fPIC", "-shared", "-fvisibility=hidden",
           "-I", sysconfig.get_paths()["include"], "-I", INCLUDE,
           os.path.join(CSRC, "argreduce_pyfast.c"), "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"fast-call binding failed ({proc.returncode}):\n{proc.stderr[-4000:]}")
    os.replace(out + ".tmp", out)
    return out


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the shared library."""
    objdir = os.path.join(os.path.dirname(out), "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in flags() if f != "-shared"]
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [hipcc(), *compile_flags, *(extra or []), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
    failed = []
    for src, proc in procs:
        _, err = proc.communicate()
        if proc.returncode != 0:
            failed.append(f"{os.path.basename(src)} ({proc.returncode}):\n{err[-6000:]}")
    if failed:
        raise RuntimeError("hipcc failed: " + "\n".join(failed))
    cmd = [hipcc(), *flags(), *(extra or []), *objs, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed ({proc.returncode}):\n{proc.stderr[-8000:]}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_fast_binding(verbose="-v" in sys.argv))
