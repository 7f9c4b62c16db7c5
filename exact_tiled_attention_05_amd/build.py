"""Build libfa.so (the gfx950 attention kernels and their C ABI) in-tree with hipcc.

Usage: python -m exact_tiled_attention_05_amd.build   (or __graft_entry__.build()).
Always recompiles every source; objects go to _build/ at the repository root.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

HIP_SOURCES = ["fa_fwd_bf16.hip", "fa_fwd_f32.hip", "fa_decode.hip", "fa_combine.hip",
               "fa_bwd_bf16.hip", "fa_fwd_fp8.hip"]
CPP_SOURCES = ["fa_api.cpp"]

COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}"]
# Device code is built without packed-fp32 instructions.
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-ffp-contract=fast"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=None, out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every source and link `out` (default: the in-tree libfa.so)."""
    os.makedirs(build_dir, exist_ok=True)
    hipcc = _hipcc()
    extra = list(extra_flags or [])
    jobs = []
    for s in HIP_SOURCES:
        obj = os.path.join(build_dir, s + ".o")
        jobs.append([hipcc, *COMMON, *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, s), "-o", obj])
    for s in CPP_SOURCES:
        obj = os.path.join(build_dir, s + ".o")
        jobs.append([hipcc, *COMMON, *extra, "-c", os.path.join(CSRC, s), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [j[-1] for j in jobs]
    tmp = out + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    if out == LIB:
        build_c_example()
        build_serial_copies(objs, build_dir, extra)
    return out


# Sources whose LDS pipelines have a single-buffered verification form
# (FA_SERIAL_COPIES: every tile copied, waited for and fenced by barriers on
# both sides, no copy overlapping compute).
SERIAL_SOURCES = ["fa_fwd_bf16.hip", "fa_fwd_fp8.hip", "fa_bwd_bf16.hip"]
SERIAL_LIB = os.path.join(ROOT, "tests", "hazard", "libfa_serial_copies.so")


def build_serial_copies(objs, build_dir=BUILD, extra=()) -> str:
    """A verification copy of the library (tests only): the sources in SERIAL_SOURCES
    rebuilt with FA_SERIAL_COPIES, linked with the other objects of the main build.
    The GPU hazard test checks that it gives the same bits as libfa.so."""
    hipcc = _hipcc()
    sdir = os.path.join(build_dir, "serial_copies")
    os.makedirs(sdir, exist_ok=True)
    os.makedirs(os.path.dirname(SERIAL_LIB), exist_ok=True)
    jobs, swap = [], {}
    for src in SERIAL_SOURCES:
        obj = os.path.join(sdir, src + ".o")
        jobs.append([hipcc, *COMMON, *HIP_FLAGS, *extra, "-DFA_SERIAL_COPIES", "-c",
                     os.path.join(CSRC, src), "-o", obj])
        swap[os.path.join(build_dir, src + ".o")] = obj
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        list(ex.map(_run, jobs))
    tmp = SERIAL_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[swap.get(o, o) for o in objs],
          "-o", tmp])
    os.replace(tmp, SERIAL_LIB)
    return SERIAL_LIB


C_EXAMPLE_DIR = os.path.join(ROOT, "tests", "c_abi")
C_EXAMPLE = os.path.join(C_EXAMPLE_DIR, "fa_c_example")


def build_c_example() -> str:
    """Compile the plain C consumer of the C ABI (tests/c_abi/fa_c_example.c) with gcc,
    linked against the in-tree libfa.so and the HIP runtime."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    _run(["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
          f"-I{rocm}/include", f"-I{INCLUDE}", os.path.join(C_EXAMPLE_DIR, "fa_c_example.c"),
          f"-L{PKG}", "-lfa", f"-L{rocm}/lib", "-lamdhip64", "-lm",
          "-Wl,-rpath,$ORIGIN/../../exact_tiled_attention_05_amd", f"-Wl,-rpath,{rocm}/lib",
          "-o", C_EXAMPLE])
    return C_EXAMPLE


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
