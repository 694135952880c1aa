"""Build libsattn.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: python -m sparse_self_attention_amd.build   (or call build()).
Objects go to sparse_self_attention_amd/_build/, the library to sparse_self_attention_amd/libsattn.so and the
benchmark's MFMA rate probe to sparse_self_attention_amd/libsattn_probe.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsattn.so")
PROBE_LIB = os.path.join(PKG, "libsattn_probe.so")     # the benchmark's MFMA rate probe
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_SOURCES = ["attn_fwd.hip", "mask.hip", "cached_mask.hip", "fp8_attn.hip", "util.hip", "noalloc.hip"]
CXX_SOURCES = ["api.cpp", "mask_sizes.cpp"]

# Packed fp32 VALU forms are kept out of the generated code.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include")]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + msg)
    return msg


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libsattn.so; returns the library path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    jobs = []
    for s in HIP_SOURCES:
        o = os.path.join(OUT_DIR, s + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
    for s in CXX_SOURCES:
        o = os.path.join(OUT_DIR, s + ".o")
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        logs = list(ex.map(_run, jobs))
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    logs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    # the benchmark's MFMA rate probe: a library of its own, outside the attention ABI
    probe_o = os.path.join(OUT_DIR, "probe_mfma.hip.o")
    logs.append(_run([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "probe_mfma.hip"), "-o", probe_o]))
    logs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", probe_o, "-o", PROBE_LIB + ".tmp"]))
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
