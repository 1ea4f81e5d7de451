"""Build the HIP library librs.so in-tree for gfx950.

    python -m ssm_decode_checkpoint_amd.build        # or build() from Python

Each .hip source is compiled to an object with hipcc and the host-only C ABI
source (rs_host.cpp) with the host C++ compiler, in parallel, then linked into
ssm_decode_checkpoint_amd/librs.so. Packed-fp32 instruction selection is
switched off for device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librs.so")
PROBE_LIB = os.path.join(PKG, "librs_probe.so")   # measurement helper, separate from the decode library
SOURCES = ["rs_commit.hip", "rs_block.hip", "rs_mamba2.hip", "rs_m2_16x16.hip", "rs_m2_64x64.hip", "rs_m2_128x64.hip",
           "rs_m2_128x128.hip", "rs_gdn.hip"]

# the C ABI's host side: plain C++, no GPU header, built by the host compiler
HOST_SOURCES = ["rs_host.cpp"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
ARCH = "gfx950"
# -packed-fp32-ops: no packed fp32 instructions. The atomic optimizer is off
# because it rewrites a one-lane atomic into a wave scan that waits for every
# load in flight, which stalls the counter arrival behind the state stream.
# Matrix-core results stay in ordinary vector registers (the fold's
# accumulators are the state tile itself; the accumulation-register form
# copies them and costs occupancy).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None", "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _compile_host(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".host.o")
    cmd = [CXX, *HOST_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{CXX} failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link librs.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES) + len(HOST_SOURCES), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(jobs) as ex:
        hobjs = [ex.submit(_compile_host, s) for s in HOST_SOURCES]
        objs = list(ex.map(_compile, SOURCES)) + [h.result() for h in hobjs]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, LIB)
    probe = _compile("rs_probe.hip")
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", probe, "-o", PROBE_LIB + ".tmp"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    shutil.move(PROBE_LIB + ".tmp", PROBE_LIB)
    if verbose:
        print(f"built {LIB}")
        print(f"built {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
