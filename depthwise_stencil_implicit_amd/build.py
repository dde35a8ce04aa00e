"""Build ``libmiconv.so`` in-tree: hipcc for the gfx950 kernels, g++ for the
host-only binding/planner, one shared library with only the C ABI exported.

    python -m depthwise_stencil_implicit_amd.build [-v]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmiconv.so")
PROBE_SRC = os.path.join(PKG, "probe", "probe.hip")
PROBE_LIB = os.path.join(PKG, "probe", "libmiconv_probe.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
             # Packed fp32 VALU ops (v_pk_*_f32) stay off in every kernel.
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics", "-Wno-unused-result"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra",
             "-Wno-unused-parameter", f"-I{ROCM}/include", "-D__HIP_PLATFORM_AMD__"]


def _sources():
    hip, cpp = [], []
    for f in sorted(os.listdir(CSRC)):
        p = os.path.join(CSRC, f)
        if f.endswith(".hip"):
            hip.append(p)
        elif f.endswith(".cpp"):
            cpp.append(p)
    return hip, cpp


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [os.path.join(ROCM, "bin", "hipcc"), *HIP_FLAGS, f"-I{INCLUDE}", "-c", src, "-o", obj]
    else:
        cmd = ["g++", *CXX_FLAGS, f"-I{INCLUDE}", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise and verbose:
        print("\n".join(noise), file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source and link ``libmiconv.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    hip, cpp = _sources()
    jobs = jobs or min(8, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), hip + cpp))
    tmp = LIB + ".tmp"
    cmd = [os.path.join(ROCM, "bin", "hipcc"), "-shared", "-fPIC", f"--offload-arch={ARCH}",
           *objs, "-o", tmp, f"-L{ROCM}/lib", "-lamdhip64"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_probe(verbose)
    return LIB


def build_probe(verbose: bool = False) -> str:
    """The measurement probes (MFMA issue rate, LDS read bandwidth): a small
    library of their own, loaded only by the benchmark's probe modes."""
    tmp = PROBE_LIB + ".tmp"
    # MFMA results in VGPRs: with accumulation registers the allocator moves
    # the probe's accumulators between rounds, which would time the moves.
    cmd = [os.path.join(ROCM, "bin", "hipcc"), *HIP_FLAGS, "-mllvm", "-amdgpu-mfma-vgpr-form", "-shared", PROBE_SRC,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
