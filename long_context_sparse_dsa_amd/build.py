"""Build libdsa.so (gfx950) in-tree with hipcc.

Every HIP source is compiled with packed-fp32 instruction selection disabled
(the compiler may otherwise form v_pk_* fp32 ops from scalar or float2 code)
and with strict aliasing off, because the kernels view LDS and global buffers
through several vector types.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdsa.so")
PROBE_SRC = os.path.join(PKG, "probe", "peaks.hip")
PROBE_LIB = os.path.join(PKG, "libdsa_peaks.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = os.environ.get("DSA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fno-strict-aliasing",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    # the host pass does not know the GPU target feature; everything else is shown
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(ln for ln in r.stderr.splitlines() if noise not in ln)
    if msg.strip():
        sys.stderr.write(msg + "\n")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """libdsa.so (the DSA path) and libdsa_peaks.so (the benchmark's peak
    probes, a separate library)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        fut_probe = ex.submit(_compile, PROBE_SRC)
        objs = list(ex.map(_compile, srcs))
        probe_obj = fut_probe.result()
    _link(objs, LIB)
    _link([probe_obj], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
