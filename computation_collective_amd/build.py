"""Build libhocf.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every source is compiled by hipcc into its own object (in parallel), then
linked into ``computation_collective_amd/libhocf.so``.  The device code is
built with packed-fp32 instructions disabled (plain fp32 arithmetic only).

The trace build, ``libhocf_trace.so``, is the same library with HOCF_TRACE
defined in the sources that use it (the GEMM + ReduceScatter / AllReduce
kernel records per-iteration timestamps into its workspace; see
csrc/trace.hpp); the other objects are shared."""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libhocf.so")
TRACE_LIB = os.path.join(HERE, "libhocf_trace.so")
SOURCES = ["abi.cpp", "gemm_rs.hip", "gemv_ar.hip", "ag_gemm.hip", "embbag_a2a.hip", "gemm_a2a.hip",
           "a2a_gemm.hip"]
TRACE_SOURCES = ["abi.cpp", "gemm_rs.hip"]   # the sources HOCF_TRACE changes
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libhocf.so")


def flags() -> list[str]:
    return ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Wall", "-Wno-unused-function", "-I", INCLUDE,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, verbose: bool, trace: bool = False) -> str:
    out = os.path.join(BUILD, "trace") if trace else BUILD
    obj = os.path.join(out, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags() + (["-DHOCF_TRACE=1"] if trace else []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature and says so: harmless
    noise = [l for l in r.stderr.splitlines() if l.strip() and "packed-fp32-ops" not in l
             and "not a recognized feature" not in l]
    if verbose and noise:
        print("\n".join(noise))
    return obj


def _link(objs: list[str], lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Both libraries; returns the product library's path."""
    os.makedirs(os.path.join(BUILD, "trace"), exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + [(s, True) for s in TRACE_SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs))
    plain = dict(zip(SOURCES, objs[:len(SOURCES)]))
    traced = dict(zip(TRACE_SOURCES, objs[len(SOURCES):]))
    _link([plain[s] for s in SOURCES], LIB, verbose)
    _link([traced.get(s, plain[s]) for s in SOURCES], TRACE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
