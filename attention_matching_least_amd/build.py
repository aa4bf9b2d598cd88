"""Builds libamc.so (HIP, gfx950) in-tree, and the peak probe ``amc_peaks``.

Each source is compiled to an object under ``_build/`` in parallel, then the
objects are linked into ``attention_matching_least_amd/libamc.so``.
``amc_peaks`` (peaks/peaks.hip) measures the MFMA, vector and HBM rates the
roofline figures are compared with.
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
LIB = os.path.join(PKG, "libamc.so")
PEAKS_SRC = os.path.join(PKG, "peaks", "peaks.hip")
PEAKS = os.path.join(PKG, "amc_peaks")

SOURCES = ["amc_api.cpp", "k_phi.hip", "k_select.hip", "k_nnls.hip", "k_nnls_g.hip", "k_nnls_qr.hip", "k_ols.hip"]

ARCH = os.environ.get("AMC_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-I", INCLUDE,
    "-I", CSRC,
    # packed fp32 instructions are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    res = subprocess.run([HIPCC, *COMMON, "-x", "hip", PEAKS_SRC, "-o", PEAKS + ".tmp"], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for the peak probe:\n{res.stdout}\n{res.stderr}")
    os.replace(PEAKS + ".tmp", PEAKS)
    if verbose:
        print(f"built {LIB} and {PEAKS}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
