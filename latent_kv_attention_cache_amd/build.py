"""Build the HIP shared library ``libvmla.so`` in-tree for gfx950.

Run ``python -m latent_kv_attention_cache_amd.build`` (or call ``build()``).
Objects go to ``_build/`` at the repository root; the library is written next
to this file, where the binding loads it from.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libvmla.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["vmla_api.cpp", "append.hip", "qprologue.hip", "latent_attn.hip", "latent_attn_wide.hip",
           "mixer_gemm.hip", "explicit_attn.hip", "noalloc.hip"]
# Per-source extra flags. The attention kernel never reads NaNs (slots past the
# valid prefix are not loaded), so max() needs no NaN canonicalization.
EXTRA_FLAGS = {"latent_attn.hip": ["-fno-honor-nans"], "latent_attn_wide.hip": ["-fno-honor-nans"]}
# The matrix-core peak probe (the measured roofline reference of bench.py) is
# its own library, outside the C ABI of libvmla.so.
PROBE_SOURCE = "peak_probe.hip"
PROBE_PATH = os.path.join(PKG, "libvmla_probe.so")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay disabled on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source, link ``libvmla.so`` and the peak-probe
    library ``libvmla_probe.so``; returns the path of ``libvmla.so``."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES + [PROBE_SOURCE]))
    _link(objs[:-1], LIB_PATH, verbose)
    _link(objs[-1:], PROBE_PATH, verbose)
    return LIB_PATH


def _link(objs, path, verbose):
    tmp = path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(path)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
