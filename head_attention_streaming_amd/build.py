"""Compile libstreamattn.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Usage: python -m head_attention_streaming_amd.build
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
LIB = os.path.join(PKG, "libstreamattn.so")
# The same library with the attention kernels built in their LDS check variant (SA_LDS_CHECK=1:
# single-buffered K/V tiles, extra barriers); the tests compare its outputs with LIB's bit for bit.
LIB_LDS_CHECK = os.path.join(PKG, "libstreamattn_ldscheck.so")
SOURCES = ["attn_fwd.hip", "qk_norm_rope.hip", "kv_cache.hip", "capi.hip"]
# Per-source extra flags. The attention kernel assumes finite inputs (NaN in q/k/v is outside its
# contract), which lets the compiler fuse the row-maximum tree into v_max3_f32.
EXTRA = {"attn_fwd.hip": ["-fno-honor-nans"]}
ARCH = "gfx950"

# Packed-fp32 VALU forms are switched off for all device code (hipcc's host pass reports the
# feature as unknown; that warning is harmless).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(src: str, obj: str, defines=()) -> None:
    cmd = [_hipcc(), *FLAGS, *EXTRA.get(src, []), *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libstreamattn.so, and its LDS check variant
    libstreamattn_ldscheck.so (attention kernels built with SA_LDS_CHECK=1); returns LIB."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    check_obj = os.path.join(objdir, "attn_fwd_ldscheck.o")
    jobs = [(s, o, ()) for s, o in zip(SOURCES, objs)] + [("attn_fwd.hip", check_obj, ("-DSA_LDS_CHECK=1",))]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        list(ex.map(lambda j: _compile(*j), jobs))
    _link(objs, LIB)
    _link([check_obj if s == "attn_fwd.hip" else o for s, o in zip(SOURCES, objs)], LIB_LDS_CHECK)
    if verbose:
        print(f"built {LIB} and {LIB_LDS_CHECK}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
