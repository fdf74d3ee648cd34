"""Build libsparge.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m block_sparse_attention_softmax_amd.build

Every translation unit under csrc/ is compiled with hipcc for gfx950 only and
linked into block_sparse_attention_softmax_amd/libsparge.so; the measurement
probe under csrc/probe/ becomes libsparge_probe.so beside it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsparge.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


PROBE_SRC = os.path.join(CSRC, "probe", "ceilings.hip")
PROBE_LIB = os.path.join(PKG, "libsparge_probe.so")


def build_probe(verbose: bool = True) -> str:
    """The measurement probe (a dense-MFMA ceiling kernel the benchmark runs
    beside the attention path; not part of the library's ABI)."""
    obj = _compile(PROBE_SRC)
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", obj, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe link failed:\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(len(srcs), 8)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    # resolve every symbol now: a missing kernel stub fails here, not at first use
    import ctypes
    ctypes.CDLL(tmp, mode=os.RTLD_NOW)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_probe(verbose)
    return LIB


if __name__ == "__main__":
    build()
